// MLA partial attention with bf16 MFMA: every query head of a request shares one latent KV
// row per token (576 = 512 latent + 64 rope dims; the value is the first 512 dims).
//
// A workgroup is one stream-K worker and holds all query heads of a request, so every KV
// byte is read from HBM exactly once. Each wave owns 16 heads. Per 32-token tile:
//   - the tile (32 rows x 1152 B) is copied HBM -> LDS with global_load_lds_dwordx4 (no
//     register staging), double-buffered so the next tile streams in while this one is used;
//   - S^T[16 tok x 16 heads] = K[16 x 576] . Q^T[576 x 16] for the two 16-row subtiles
//     (2 x 18 v_mfma_f32_16x16x32_bf16; K rows from LDS as the A operand, the wave's Q slice
//     resident in registers as B);
//   - online softmax per head: a lane holds 8 scores of one head, two shuffles reach the
//     other three lanes of that head;
//   - O^T[512 x 16] += V^T[512 x 32] . P^T[32 x 16]  (32 M tiles; V = the first 512 dims of
//     the same LDS tile, read transposed with ds_read_b64_tr_b16; P from registers, split
//     into a bf16 high part and a bf16 remainder, two MFMAs).
//
// LDS tile layout (36.5 KB): region A = dims 0..511 of the 32 rows, one 1 KB row per DMA
// instruction, rows padded to 1056 B; region B = dims 512..575, 128 B per row with the 16-byte
// chunks XOR-swizzled by row. MFMA row m of a 16-row subtile is token pi(m), where
// pi(8c + 4h + e) = 8c + h + 2e: the K reads of 8 consecutive MFMA rows then touch 8
// different 16-byte bank groups, and each transposed V read (4 MFMA rows e = 0..3) reads
// rows 2 apart, whose 32-byte pieces tile 128 bytes of banks without overlap.
#include "mla_common.h"

namespace dcp {

constexpr int kMlaTile = 32;
constexpr int kMlaRowA = 1056;                    // LDS bytes per row, region A (dims 0..511)
constexpr int kMlaRowB = 128;                     // LDS bytes per row, region B (dims 512..575)
constexpr int kMlaRegionB = kMlaTile * kMlaRowA;  // offset of region B
constexpr int kMlaTileBytes = kMlaRegionB + kMlaTile * kMlaRowB;

template <int NW>  // waves per workgroup; 16 heads per wave, Hq = 16 * NW
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_mfma_kernel(AttnArgs a, const char* __restrict__ zero_row, const int32_t* __restrict__ only) {
  __shared__ __attribute__((aligned(1024))) char lds[2][kMlaTileBytes];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int n = lane & 15;        // head within the wave; also the MFMA row this lane loads
  const int gq = lane >> 4;       // lane quarter (k-slice of the operand layouts)
  const int32_t w = blockIdx.x;
  if (w >= a.P) return;
  if (only != nullptr && only[w] == 0) return;  // recomputation pass: marked workers only
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  const char* __restrict__ Kc = (const char*)a.k;
  const int64_t T_pages = a.pre[a.U];
  const int64_t g0 = worker_begin(T_pages, a.P, w), g1 = worker_begin(T_pages, a.P, w + 1);
  if (g0 >= g1) return;
  int32_t u = find_unit(a.pre, a.U, g0);
  int64_t g = g0;
  int32_t bad = 0;
  const bool bs_pow2 = (a.bs & (a.bs - 1)) == 0;
  const int bs_shift = __builtin_ctz((unsigned)a.bs);

  // per-lane LDS offsets (bytes) within a tile buffer
  const int krow0 = tok_of_row(n);                  // K row read for MFMA row n, subtile 0
  const int ka_off = krow0 * kMlaRowA + 16 * gq;    // region A, + 64 j (+ 16 rows for subtile 1)
  const int vrow = tok_of_row(4 * gq + (n >> 2));   // V row of this lane's transposed read
  const int v_off = vrow * kMlaRowA + 8 * (n & 3);  // + 32 mt (+ 16 rows for subtile 1)

  while (g < g1) {
    while ((int64_t)a.pre[u + 1] <= g) ++u;
    const int64_t up0 = a.pre[u], up1 = a.pre[u + 1];
    const int64_t sg1 = up1 < g1 ? up1 : g1;
    const int32_t bsi = u / a.NRg, rg = u - bsi * a.NRg;  // (request, shard), row group
    const int32_t b = bsi / a.S;
    const int64_t ta = a.ubounds[2 * bsi], te = a.ubounds[2 * bsi + 1];
    const int64_t pa = ta / a.bs;
    int64_t t0 = (pa + (g - up0)) * a.bs, t1 = (pa + (sg1 - up0)) * a.bs;
    if (t0 < ta) t0 = ta;
    if (t1 > te) t1 = te;
    const bool whole = (g == up0) && (sg1 == up1);
    const bool first = (g == g0);
    const int32_t* brow = a.block_table + (int64_t)b * a.max_blocks;

    // Block id of the page holding token tile + (lane & 31), read one tile ahead of its use:
    // the load's wait then falls after the previous tile's barrier, when nothing else is in
    // flight.
    // Token positions fit in 32 bits (max_blocks_per_seq * block_size <= INT32_MAX).
    const int32_t t0i = (int32_t)t0, t1i = (int32_t)t1;
    auto page_of = [&](int32_t tile) -> int32_t {
      const int32_t t = tile + (lane & 31);
      const int32_t tc = t < t1i ? t : t1i - 1;
      return brow[bs_pow2 ? (tc >> bs_shift) : tc / a.bs];
    };
    int32_t blk_next = page_of(t0i);

    // A wave copies region-A rows wv + k NW (k < kRows) of each tile. Inside the tile loop it
    // queues half of them before the scores and the other half after: a wave that queues a
    // whole tile at once stalls on the memory pipeline's back-pressure instead of computing.
    // The rows' source addresses are wave-uniform and held in scalar registers in between.
    constexpr int kRows = kMlaTile / NW;
    uint64_t row_src[kRows];
    uint64_t rbase = 0;      // one-page tiles: source of row 0
    uint32_t rstride = 0;    // one-page tiles: bytes between rows (0 for the zero row)
    int32_t rlast = 0;       // one-page tiles: last row before t1 (later rows repeat it)
    int32_t one = 0;         // wave-uniform: the pending tile lies in one page
    uint32_t base_pend = 0;
    auto issue_rows = [&](int k0, int k1) {
      if (one) {
#pragma unroll
        for (int k = k0; k < k1; ++k) {
          const int r = wv + k * NW;
          const uint32_t rr = (uint32_t)(r < rlast ? r : rlast);
          dma16((const char*)(rbase + (uint64_t)(rr * rstride)) + 16 * lane,
                base_pend + r * kMlaRowA);
        }
      } else {
#pragma unroll
        for (int k = k0; k < k1; ++k)
          dma16((const char*)row_src[k] + 16 * lane, base_pend + (wv + k * NW) * kMlaRowA);
      }
    };
    // Queue the copy of tile [tile, tile + 32) into buffer `buf` (all region-A rows, or the
    // first half of them with the rest left to issue_rows); returns the valid-token mask.
    auto issue_tile = [&](int32_t tile, int buf, bool all) -> uint32_t {
      const int32_t blk = blk_next;
      if (tile + kMlaTile < t1i) blk_next = page_of(tile + kMlaTile);
      const uint32_t base = lds_u32(&lds[buf][0]);
      base_pend = base;
      one = bs_pow2 ? ((tile >> bs_shift) == ((tile + kMlaTile - 1) >> bs_shift))
                    : (tile / a.bs == (tile + kMlaTile - 1) / a.bs);
      if (one) {
        // rows tile .. tile + 31 lie in one page; rows past t1 repeat the last valid row (the
        // page's later slots may hold anything, and a NaN there would survive its zero weight
        // in the value product)
        const int32_t blk1 = __builtin_amdgcn_readfirstlane(blk);
        const bool page_ok = blk1 >= 0 && blk1 < a.num_blocks;
        const uint32_t slot0 = bs_pow2 ? (uint32_t)(tile & (a.bs - 1)) : (uint32_t)(tile % a.bs);
        rbase = page_ok ? (uint64_t)Kc + ((uint64_t)(uint32_t)blk1 * (uint32_t)a.bs + slot0) *
                                             (kMlaDqk * 2)
                        : (uint64_t)zero_row;
        rstride = page_ok ? kMlaDqk * 2 : 0;
        rlast = t1i - 1 - tile;
        if (!page_ok) bad = 1;
        const uint32_t m = (uint32_t)__ballot(page_ok && lane < kMlaTile && tile + lane < t1i);
        issue_rows(0, all ? kRows : kRows / 2);
        for (int kk = wv; kk < 4; kk += NW) {
          const int r = 8 * kk + (lane >> 3);
          const uint32_t rr = (uint32_t)(r < rlast ? r : rlast);
          const uint64_t ra = rbase + (uint64_t)(rr * rstride);
          dma16((const char*)ra + 1024 + 16 * ((lane & 7) ^ swz_b(r)),
                base + kMlaRegionB + kk * 1024);
        }
        return m;
      }
      uint64_t rowaddr = (uint64_t)zero_row;
      bool valid = false;
      if (lane < kMlaTile) {
        const int32_t t = tile + lane;
        const int32_t tc = t < t1i ? t : t1i - 1;
        const bool page_ok = blk >= 0 && blk < a.num_blocks;
        // row index < num_blocks * block_size rows of 1152 B: below 2^31 for any pool that
        // fits in device memory
        const uint32_t slot = bs_pow2 ? (uint32_t)(tc & (a.bs - 1)) : (uint32_t)(tc % a.bs);
        const uint32_t row = (uint32_t)blk * (uint32_t)a.bs + slot;
        if (page_ok)
          rowaddr = (uint64_t)Kc + (uint64_t)row * (kMlaDqk * 2);
        else
          bad = 1;
        valid = page_ok && t < t1i;
      }
      const uint32_t mask = (uint32_t)__ballot(valid);
#pragma unroll
      for (int k = 0; k < kRows; ++k) row_src[k] = readlane_u64(rowaddr, wv + k * NW);
      issue_rows(0, all ? kRows : kRows / 2);
      for (int kk = wv; kk < 4; kk += NW) {
        // lane covers row 8 kk + lane / 8: pick its address among the eight rows' addresses
        uint64_t ra = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint64_t aj = readlane_u64(rowaddr, 8 * kk + j);
          ra = ((lane >> 3) == j) ? aj : ra;
        }
        const int r = 8 * kk + (lane >> 3);
        dma16((const char*)ra + 1024 + 16 * ((lane & 7) ^ swz_b(r)),
              base + kMlaRegionB + kk * 1024);
      }
      return mask;
    };

    // This wave's 16 query rows (head h of query token jq; 16 | Hq, so one token per wave)
    // and the last context position they may see; rows past R are padding and not stored.
    int32_t jq = 0;
    const int32_t rho = unit_row(a, 0, rg, 16 * wv + n, &jq);
    const bool row_ok = rho >= 0;
    const int32_t lim = a.Rs == a.Hq ? INT32_MAX
                                  : __builtin_amdgcn_readfirstlane(a.qend[b] + a.j0 + jq);
    // the wave's Q slice as the B operand: lane holds q[row][32j + 8gq .. +8]
    bf16x8 qop[kMlaDqk / 32];
    {
      const uint16_t* qrow = Q + call_row(a, b, row_ok ? rho : 0) * kMlaDqk + 8 * gq;
#pragma unroll
      for (int j = 0; j < kMlaDqk / 32; ++j)
        qop[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * j));
    }

    f32x4 acc[kMlaDv / 16];
#pragma unroll
    for (int i = 0; i < kMlaDv / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    uint32_t mask_next = issue_tile(t0i, 0, true);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): the copies of the first tile
    __syncthreads();
    int cur = 0;
    for (int32_t tile = t0i; tile < t1i; tile += kMlaTile) {
      // valid tokens, less those past the rows' own position (several query tokens)
      const int32_t dl = lim - tile;
      const uint32_t mask =
          mask_next & (dl < 0 ? 0u : dl >= kMlaTile - 1 ? 0xFFFFFFFFu : (2u << dl) - 1u);
      constexpr int kQ = kRows / 2;  // rows queued before the scores
      const bool more = tile + kMlaTile < t1i;
      if (more) mask_next = issue_tile(tile + kMlaTile, cur ^ 1, false);
      const char* tb = &lds[cur][0];

      // S^T = K . Q^T for the two 16-row subtiles
      f32x4 s[2];
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        s[at] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kr = 16 * at + krow0;
        const char* pa_ = tb + ka_off + at * 16 * kMlaRowA;
        const char* pb_ = tb + kMlaRegionB + kr * kMlaRowB;
#pragma unroll
        for (int j = 0; j < kMlaDqk / 32; ++j) {
          const char* p = (j < 16) ? pa_ + 64 * j
                                   : pb_ + 16 * ((4 * (j - 16) + gq) ^ swz_b(kr));
          const bf16x8 kop = __builtin_bit_cast(bf16x8, *(const u32x4*)p);
          s[at] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[j], s[at], 0, 0, 0);
        }
      }

      if (more) issue_rows(kQ, kRows);
      // online softmax; s[at][i] is MFMA row 4gq + i of subtile at (token 16at + pi(4gq + i))
      float x[8];
      float tmax = kNegInf;
#pragma unroll
      for (int at = 0; at < 2; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * at + tok_of_row(4 * gq + i);
          const float v = ((mask >> tok) & 1u) ? s[at][i] * a.scale_log2 : kNegInf;
          x[4 * at + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = quad_max(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      float psum = 0.f;
      bf16x8 phi, plo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = (x[k] == kNegInf) ? 0.f : fast_exp2(x[k] - m_new);
        psum += p;
        const __bf16 hi = (__bf16)p;
        phi[k] = hi;
        plo[k] = (__bf16)(p - (float)hi);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int i = 0; i < kMlaDv / 16; ++i) acc[i] *= alpha;
      }

      // O^T += V^T . P^T; slots 0..3 are subtile-0 rows 4gq + e, slots 4..7 subtile-1 rows
      {
        const char* vb = tb + v_off;
#pragma unroll
        for (int mt = 0; mt < kMlaDv / 16; ++mt) {
          const bf16x8 vop = mla_tr_pair(vb + 32 * mt, vb + 16 * kMlaRowA + 32 * mt);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, acc[mt], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): the next tile's copies landed
      __syncthreads();
      cur ^= 1;
    }

    // finalise this segment: l over the four lanes of head n
    const float l = quad_sum(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst_o;
    float* dst_l;
    if (whole) {
      dst_o = a.part_o + part_row(a, bsi, rho) * kMlaDv;
      dst_l = a.part_lse + part_row(a, bsi, rho);
    } else {
      const int32_t slot = piece_slot(w, first);
      dst_o = a.piece_o + ((int64_t)slot * a.Ru + 16 * wv + n) * kMlaDv;
      dst_l = a.piece_lse + (int64_t)slot * a.Ru + 16 * wv + n;
    }
    if (row_ok) {
#pragma unroll
      for (int mt = 0; mt < kMlaDv / 16; ++mt)
        *(f32x4*)(dst_o + 16 * mt + 4 * gq) = acc[mt] * inv;
      if (gq == 0) *dst_l = l > 0.f ? (m_run + fast_log2(l)) * kLn2 : kNegInf;
    }
    g = sg1;
  }
  if (bad) atomicOr(a.flags, kFlagBadBlock);
}

int32_t mla_mfma_workers(int device, int32_t Ru, int32_t max_workers) {
  // 64 rows: one 12-wave ring workgroup per CU (157 KB of LDS); 128 rows: one 8-wave fp16
  // workgroup per CU. Otherwise LDS (2 x 36.5 KB per workgroup) allows two resident
  // workgroups per CU and registers two waves per SIMD, so two workgroups fit while a
  // workgroup has at most four waves.
  const int nw = Ru / 16;
  const int per_cu = (Ru == 64 || nw > 4) ? 1 : 2;
  int32_t p = mla_cus(device) * per_cu;
  return p < max_workers ? p : max_workers;
}

hipError_t launch_mla_mfma(const AttnArgs& a, hipStream_t stream) {
  const char* zr = a.zero_row;
  // 64 rows: the ring kernel, which rescales in place when a reference is raised
  if (a.Ru == 64) return launch_mla_ring(a, stream);
  if (a.Ru == 128) {
    // pairs of waves share an fp16 value product; workers whose values fp16 cannot hold are
    // recomputed in bf16 by the 16-rows-per-wave kernel (same worker count)
    const hipError_t e = launch_mla_pair16(a, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((mla_mfma_kernel<8>), dim3(a.P), dim3(512), 0, stream, a, zr,
                       (const int32_t*)a.redo);
    return hipGetLastError();
  }
  const int32_t* none = nullptr;
  switch (a.Ru / 16) {
    case 1: hipLaunchKernelGGL((mla_mfma_kernel<1>), dim3(a.P), dim3(64), 0, stream, a, zr, none); break;
    case 2: hipLaunchKernelGGL((mla_mfma_kernel<2>), dim3(a.P), dim3(128), 0, stream, a, zr, none); break;
    case 4: hipLaunchKernelGGL((mla_mfma_kernel<4>), dim3(a.P), dim3(256), 0, stream, a, zr, none); break;
    case 8: hipLaunchKernelGGL((mla_mfma_kernel<8>), dim3(a.P), dim3(512), 0, stream, a, zr, none); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dcp
