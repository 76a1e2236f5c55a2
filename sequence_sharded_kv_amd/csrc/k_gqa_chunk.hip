// GQA partial attention, bf16, head_dim 128: units of 32 to 256 query rows of one KV head
// (one decode token's G heads padded to 32, several query tokens per request, or a prefill
// chunk in groups of 256).
//
// A workgroup of NW waves owns 32 * NW rows of one KV head and the waves share each K/V tile
// through a three-slot LDS ring filled two tiles ahead, so the shard's pages are read once per
// 32 * NW rows. Tiles hold 32 tokens, or 64 in the 8-wave instance (one workgroup per CU, so
// its 96 KB of LDS fit, and the per-tile work of the copies, the maximum and the waits is
// spread over twice the scores). Per 32 tokens of a tile, wave w (rows 32 w .. 32 w + 31):
//   S[32 tok x 32 rows] = K[32 x 128] . Q^T[128 x 32]   8 x v_mfma_f32_32x32x16_bf16, K rows
//                                                       from LDS, the rows' Q in registers;
//   weights per row against a reference max (a lane holds 16 scores of its row, the other 16
//   are in lane l ^ 32), each row masked at its own causal limit where the tile is not fully
//   visible;
//   O^T[128 x 32] += V^T[128 x 32 tok] . P[32 tok x 32 rows]   4 M blocks x 2 k steps, V read
//                                                       transposed from LDS, P as a bf16 high
//                                                       part and remainder (two MFMAs).
// The tile loop is unrolled over the ring's slots so that every LDS read is a fixed per-lane
// offset plus an immediate. Two waves share each SIMD.
//
// Tile layout: per slot a K tile then a V tile, each kT rows x 256 B; 16-byte chunk c of row r
// sits at position c ^ sw(r), sw(r) = ((r & 3) << 2) | ((r >> 2) & 3). A 256-byte row spans all
// 64 banks once, so a chunk's banks depend on its position only; the swizzle spreads the K
// reads (32 rows, one chunk each) and the transposed V reads over distinct banks. One copy
// instruction fills 4 rows (lane i: row 4k + i / 16, position i % 16, fetching chunk
// (i % 16) ^ sw(row)).
#include "device_common.h"

#include <type_traits>

namespace dcp {

namespace gchunk {
constexpr int kD = 128;
constexpr int kRowB = kD * 2;           // 256 bytes per token row
constexpr int kSlots = 3;
__device__ __forceinline__ int sw(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

__device__ __forceinline__ bf16x8 tr_pair(const char* lo, const char* hi) {
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lo);
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)hi);
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  i16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, z);
}
}  // namespace gchunk

template <int NW, int kT>  // waves per workgroup (32 rows each); tokens per tile (32 or 64)
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
gqa_chunk_kernel(AttnArgs a) {
  using namespace gchunk;
  static_assert(kT == 32 || kT == 64, "tile of 32 or 64 tokens");
  constexpr int kH = kT / 32;               // 32-token halves of a tile
  constexpr int kTB = kT * kRowB;           // one K or V tile
  constexpr int kSB = 2 * kTB;              // K tile then V tile
  constexpr int kCp = kT / 4 / NW;          // copy instructions per wave per K (or V) tile
  constexpr int kDma = 2 * kCp;             // copies per wave per tile
  __shared__ __attribute__((aligned(1024))) char lds[kSlots * kSB];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;      // lane half: k slice of the 32x32x16 operand layouts
  const int c32 = lane & 31;    // operand row / column index
  const int32_t w = blockIdx.x;
  if (w >= a.P) return;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  const char* __restrict__ Kc = (const char*)a.k;
  const char* __restrict__ Vc = (const char*)a.v;
  const int64_t T_pages = a.pre[a.U];
  const int64_t g0 = worker_begin(T_pages, a.P, w), g1 = worker_begin(T_pages, a.P, w + 1);
  if (g0 >= g1) return;
  int32_t u = find_unit(a.pre, a.U, g0);
  int64_t gg = g0;
  int32_t bad = 0, raised = 0;
  const bool bs_pow2 = (a.bs & (a.bs - 1)) == 0;
  const int bs_shift = __builtin_ctz((unsigned)a.bs);
  const uint32_t lds0 = lds_u32(&lds[0]);

  // Per-lane LDS byte offsets within a slot, fixed for the kernel; a slot's base, a tile's
  // second 32-token half (8192 B further) and the value product's second 16-token k step
  // (4096 B) are immediates.
  //   score reads: row c32, chunk (2 ks + g) ^ sw(c32);
  //   transposed value reads: 16-lane group q4, lane L reads rows 4 (q4 >> 1) + (L >> 2) (+ 8),
  //   chunk 4 mt + 2 (q4 & 1) + ((L & 3) >> 1), byte 8 (L & 1) of the chunk. sw(r) depends on
  //   r mod 16 only.
  uint32_t koff[8], voff[8];
  {
    const int fq = sw(c32);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) koff[ks] = c32 * kRowB + 16 * ((2 * ks + g) ^ fq);
    const int q4 = lane >> 4, L = lane & 15;
    const int vr = 4 * (q4 >> 1) + (L >> 2);
    const int vc = 2 * (q4 & 1) + ((L & 3) >> 1);
    const int vw = 8 * (L & 1);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int r = vr + 8 * hf;
        voff[2 * mt + hf] = kTB + r * kRowB + vw + 16 * ((vc + 4 * mt) ^ sw(r));
      }
#pragma unroll
    for (int q = 0; q < 8; ++q) asm volatile("" : "+v"(koff[q]), "+v"(voff[q]));
  }

  while (gg < g1) {
    while ((int64_t)a.pre[u + 1] <= gg) ++u;
    const int64_t up0 = a.pre[u], up1 = a.pre[u + 1];
    const int64_t sg1 = up1 < g1 ? up1 : g1;
    const int32_t per_bs = a.Hkv * a.NRg;
    const int32_t bsi = u / per_bs, hsub = u - bsi * per_bs;
    const int32_t kvh = hsub / a.NRg, rg = hsub - kvh * a.NRg;
    const int32_t b = bsi / a.S;
    const int64_t ta = a.ubounds[2 * bsi], te = a.ubounds[2 * bsi + 1];
    const int64_t pa = ta / a.bs;
    int64_t t0 = (pa + (gg - up0)) * a.bs, t1 = (pa + (sg1 - up0)) * a.bs;
    if (t0 < ta) t0 = ta;
    if (t1 > te) t1 = te;
    const bool whole = (gg == up0) && (sg1 == up1);
    const bool first = (gg == g0);
    const int32_t* brow = a.block_table + (int64_t)b * a.max_blocks;
    const int32_t t0i = (int32_t)t0, t1i = (int32_t)t1;
    const int32_t ntiles = (t1i - t0i + kT - 1) / kT;  // >= 1
    auto page_idx = [&](int32_t t) -> int32_t { return bs_pow2 ? (t >> bs_shift) : t / a.bs; };
    const int32_t plast_seg = page_idx(t1i - 1);

    // this lane's query row (MFMA column c32 of the wave's 32 rows) and its causal limit
    int32_t jq = 0;
    const int32_t rho = unit_row(a, kvh, rg, 32 * wv + c32, &jq);
    const bool row_ok = rho >= 0;
    const int32_t lim = (a.Rs == a.Hq || !row_ok) ? INT32_MAX : a.qend[b] + a.j0 + jq;

    // Block ids of the segment's pages, 64 at a time: lane j holds the id of page pchunk + j.
    int32_t pchunk = -1, pid = -1;
    auto ensure_pages = [&](int32_t pfirst, int32_t plast) {
      if (pchunk < 0 || plast >= pchunk + 64) {
        pchunk = pfirst;
        const int32_t pp = pchunk + lane;
        pid = (pp <= plast_seg) ? brow[pp] : -1;
        asm volatile("" : "+v"(pid));  // keep the wait for this load inside the branch
      }
    };

    // Queue tile i into slot i % kSlots: this wave's copy instructions k = wv + NW m of the K
    // tile and of the V tile (one instruction fills rows 4k .. 4k + 3). Lane t < kT (t and
    // t + 32 for 32-token tiles) finds token tile + t's row in the caches (all ones for an
    // invalid page) with one lane permute of the page ids; each copy lane then fetches the
    // row index of its own row the same way. Returns the tile's valid-token mask.
    auto issue_tile = [&](int32_t i) -> uint64_t {
      const int32_t tile = t0i + kT * i;
      const int32_t tl = (tile + kT - 1 < t1i ? tile + kT - 1 : t1i - 1);
      ensure_pages(page_idx(tile), page_idx(tl));
      const int32_t t = tile + (kT == 64 ? lane : c32);
      const int32_t tc = t < t1i ? t : t1i - 1;
      const int32_t blk = __builtin_amdgcn_ds_bpermute(4 * (page_idx(tc) - pchunk), pid);
      const bool page_ok = blk >= 0 && blk < a.num_blocks;
      const uint32_t slot = bs_pow2 ? (uint32_t)(tc & (a.bs - 1)) : (uint32_t)(tc % a.bs);
      // row index in the caches (below 2^32 - 1 for any pool that fits in device memory), all
      // ones for an invalid page
      const uint32_t row =
          page_ok ? ((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh) * (uint32_t)a.bs + slot
                  : 0xFFFFFFFFu;
      bad |= __any(!page_ok) ? 1 : 0;
      const uint64_t mask = (uint64_t)__ballot((kT == 64 || lane < 32) && page_ok && t < t1i);
      const uint32_t base = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((i % kSlots) * kSB));
      const int sub = lane >> 4, p = lane & 15;
#pragma unroll
      for (int m = 0; m < kCp; ++m) {
        const int k = wv + NW * m;  // rows 4k .. 4k + 3
        const int r = 4 * k + sub;
        const uint32_t rr = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * r, (int)row);
        const int64_t chunk = 16 * (p ^ sw(r));
        const bool ok = rr != 0xFFFFFFFFu;
        const char* ks = ok ? Kc + (uint64_t)rr * kRowB + chunk : a.zero_row + chunk;
        const char* vs = ok ? Vc + (uint64_t)rr * kRowB + chunk : a.zero_row + chunk;
        dma16(ks, base + k * 1024);
        dma16(vs, base + kTB + k * 1024);
      }
      return mask;
    };
    auto wait_tiles = [&](int32_t later) {  // at most `later` tiles' copies in flight
      if (later >= 1)
        __builtin_amdgcn_s_waitcnt((kDma & 15) | ((kDma >> 4) << 14) | (7 << 4) | (15 << 8));
      else
        __builtin_amdgcn_s_waitcnt(0);
    };

    // Q^T as the B operand: lane holds q[row][16 ks + 8 g .. +8]
    bf16x8 qop[8];
    {
      const uint16_t* qrow = Q + call_row(a, b, row_ok ? rho : 0) * kD + 8 * g;
      u32x4 raw[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) raw[ks] = *(const u32x4*)(qrow + 16 * ks);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        asm volatile("" : "+v"(raw[ks]));  // resident: no reload inside the tile loop
        qop[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
      }
    }

    f32x16 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mt][r] = 0.f;
    // Reference max: the row's weights are exp2(s - m_ref) with m_ref set by the first tile
    // where the row sees a token (its sum and accumulator are still zero then) and raised only
    // when a later tile's maximum exceeds it by kLazy, which rescales the row's sum and
    // accumulator; otherwise the weights stay below 2^kLazy and nothing is rescaled.
    constexpr float kLazy = 16.f;
    float m_ref = kNegInf, l_run = 0.f;
    const float sl2 = a.scale_log2;

    uint32_t mlo = 0, mhi = 0;  // lane s: valid-token mask of the tile in slot s (low, high)
    int32_t issued = 0;
    auto issue_next = [&]() {
      const uint64_t m = issue_tile(issued);
      const bool mine = lane == issued % kSlots;
      mlo = mine ? (uint32_t)m : mlo;
      mhi = mine ? (uint32_t)(m >> 32) : mhi;
      ++issued;
    };
    for (int k = 0; k < kSlots - 1; ++k)
      if (issued < ntiles) issue_next();
    wait_tiles(issued - 1);
    __syncthreads();

    // one tile in slot S (a compile-time constant: the LDS offsets are immediates)
    auto body = [&](auto slot_tag, int32_t i) {
      constexpr int S = decltype(slot_tag)::value;
      if (issued < ntiles) issue_next();
      const int32_t tile = t0i + kT * i;
      const int32_t dl = lim - tile;
      const uint64_t tmask = ((uint64_t)__builtin_amdgcn_readlane(mhi, S) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane(mlo, S);
      const uint64_t cmask = dl < 0 ? 0ull : dl >= kT - 1 ? ~0ull : (2ull << dl) - 1ull;
      const uint64_t all = kT == 64 ? ~0ull : 0xFFFFFFFFull;
      const uint64_t mask = tmask & cmask & all;
      const bool full = __ballot(mask != all) == 0;  // wave-uniform
      const char* tb = lds + S * kSB;

      // S[kT tok x 32 rows] = K . Q^T, one 32-token half at a time
      f32x16 st[kH];
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        bf16x8 kbuf[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          kbuf[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(tb + 8192 * h + koff[ks]));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 kop = kbuf[ks & 3];
          if (ks + 4 < 8)
            kbuf[ks & 3] =
                __builtin_bit_cast(bf16x8, *(const u32x4*)(tb + 8192 * h + koff[ks + 4]));
          st[h] = ks == 0 ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[0], f32x16{}, 0, 0, 0)
                          : __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], st[h], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // row c32's maximum over the tile; st[h][r] is token 32 h + 8 (r / 4) + 4 g + r % 4. A
      // tile with every token visible skips the masks (their bits are formed inside the
      // masked branch only).
      float tmax = kNegInf;
      if (full) {
#pragma unroll
        for (int h = 0; h < kH; ++h)
#pragma unroll
          for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, st[h][r]);
      } else {
        uint64_t hmask = mask >> (4 * g);
        asm volatile("" : "+v"(hmask));
#pragma unroll
        for (int h = 0; h < kH; ++h)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            // a masked score becomes -inf here, so the weights below need no second mask
            const bool v = ((hmask >> (32 * h + 8 * (r >> 2) + (r & 3))) & 1ull) != 0ull;
            st[h][r] = v ? st[h][r] : kNegInf;
            tmax = fmaxf(tmax, st[h][r]);
          }
      }
      {
        auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                   false, false);
        tmax = fmaxf(__uint_as_float(s2[0]), __uint_as_float(s2[1]));
      }
      const float tm = tmax * sl2;  // the scaled maximum (scaling is monotonic)
      float rs = 1.f;
      if (m_ref == kNegInf) {
        m_ref = tm;
      } else if (tm > m_ref + kLazy) {
        rs = fast_exp2(m_ref - tm);
        m_ref = tm;
      }
      if (__ballot(rs != 1.f) != 0) {
        raised = 1;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] *= rs;
        l_run *= rs;
      }
      // Weights; a masked score is -inf and gives exp2(-inf) = 0, unless the row has seen no
      // token yet (m_ref = -inf), where every score of the tile is masked and the weights are
      // set to zero instead.
      const float nm = m_ref == kNegInf ? 0.f : -m_ref;
      // bf16 high parts packed in pairs; the remainders from the unpacked highs; k step kk of
      // half h is operand 2 h + kk
      float psum = 0.f;
      bf16x8 phi[2 * kH], plo[2 * kH];
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        u32x4 hpk[2], lpk[2];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float p0 = fast_exp2(__builtin_fmaf(st[h][2 * q], sl2, nm));
          const float p1 = fast_exp2(__builtin_fmaf(st[h][2 * q + 1], sl2, nm));
          psum += p0 + p1;
          typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
          const bf16x2 hh = {(__bf16)p0, (__bf16)p1};
          const uint32_t hbits = __builtin_bit_cast(uint32_t, hh);
          const bf16x2 lo = {(__bf16)(p0 - __uint_as_float(hbits << 16)),
                             (__bf16)(p1 - __uint_as_float(hbits & 0xFFFF0000u))};
          hpk[q >> 2][q & 3] = hbits;
          lpk[q >> 2][q & 3] = __builtin_bit_cast(uint32_t, lo);
        }
        phi[2 * h] = __builtin_bit_cast(bf16x8, hpk[0]);
        phi[2 * h + 1] = __builtin_bit_cast(bf16x8, hpk[1]);
        plo[2 * h] = __builtin_bit_cast(bf16x8, lpk[0]);
        plo[2 * h + 1] = __builtin_bit_cast(bf16x8, lpk[1]);
      }
      l_run += psum;

      // O^T[128 x 32 rows] += V^T . P over the tile's 16-token k steps
#pragma unroll
      for (int h = 0; h < kH; ++h)
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) {
          const int kk = s2 >> 2, mt = s2 & 3;
          const char* vb = tb + 8192 * h + 4096 * kk;
          const bf16x8 vop = tr_pair(vb + voff[2 * mt], vb + voff[2 * mt + 1]);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, phi[2 * h + kk], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, plo[2 * h + kk], acc[mt], 0, 0, 0);
        }
      // tile i + 1 has landed and every wave is past tile i (its slot is refilled next)
      wait_tiles(issued - (i + 2));
      __syncthreads();
    };
    for (int32_t i = 0; i < ntiles;) {
      body(std::integral_constant<int, 0>{}, i);
      if (++i >= ntiles) break;
      body(std::integral_constant<int, 1>{}, i);
      if (++i >= ntiles) break;
      body(std::integral_constant<int, 2>{}, i);
      ++i;
    }

    // finalise: l over the two lanes of row c32
    float l = l_run;
    {
      auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false,
                                                 false);
      l = __uint_as_float(s2[0]) + __uint_as_float(s2[1]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst_o;
    float* dst_l;
    if (whole) {
      dst_o = a.part_o + part_row(a, bsi, rho) * kD;
      dst_l = a.part_lse + part_row(a, bsi, rho);
    } else {
      const int32_t slot = piece_slot(w, first);
      dst_o = a.piece_o + ((int64_t)slot * a.Ru + 32 * wv + c32) * kD;
      dst_l = a.piece_lse + (int64_t)slot * a.Ru + 32 * wv + c32;
    }
    if (row_ok) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *(f32x4*)(dst_o + 32 * mt + 8 * r4 + 4 * g) =
              f32x4{acc[mt][4 * r4], acc[mt][4 * r4 + 1], acc[mt][4 * r4 + 2],
                    acc[mt][4 * r4 + 3]} * inv;
      if (g == 0) *dst_l = l > 0.f ? (m_ref + fast_log2(l)) * kLn2 : kNegInf;
    }
    gg = sg1;
  }
  if (bad && lane == 0) atomicOr(a.flags, kFlagBadBlock);
  if (__any(raised) && lane == 0) atomicOr(a.flags, kFlagRescaled);
}

int32_t gqa_chunk_workers(int device, int32_t Ru, int32_t max_workers) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  // two waves per SIMD (8 per CU) by registers, so one 8-wave workgroup (256 rows) per CU;
  // 48 KB of LDS per workgroup (96 KB for the 8-wave instance's 64-token tiles)
  const int nw = Ru / 32;
  const int by_regs = 8 / nw, by_lds = 160 / 48;
  const int per_cu = by_regs < by_lds ? by_regs : by_lds;
  int32_t p = cus * per_cu;
  return p < max_workers ? p : max_workers;
}

hipError_t launch_gqa_chunk(const AttnArgs& a, hipStream_t stream) {
  switch (a.Ru / 32) {
    case 1: hipLaunchKernelGGL((gqa_chunk_kernel<1, 32>), dim3(a.P), dim3(64), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((gqa_chunk_kernel<2, 32>), dim3(a.P), dim3(128), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((gqa_chunk_kernel<4, 32>), dim3(a.P), dim3(256), 0, stream, a); break;
    case 8: hipLaunchKernelGGL((gqa_chunk_kernel<8, 64>), dim3(a.P), dim3(512), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dcp
