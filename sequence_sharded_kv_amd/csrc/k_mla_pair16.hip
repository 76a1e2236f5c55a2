// MLA partial attention for units of 128 query rows (128 heads of one decode token, or 64
// heads x 2 tokens, 32 x 3-4, 16 x 5-8): one workgroup of 8 waves per CU, 16 rows per wave,
// the value product in fp16.
//
// Per 32-token tile (36 KB: 32 latent rows of 1152 B, double-buffered in LDS):
//   - each wave scores its own 16 rows against the tile, S^T = K . Q^T on
//     v_mfma_f32_16x16x32_bf16 (K from LDS, the rows' Q resident in registers);
//   - each wave converts 4 of the tile's 32 latent rows, value dims 0..511, from bf16 to fp16
//     into a separate 32 KB buffer of the same layout, and records the largest magnitude it
//     met;
//   - the weights p = exp2(s - m_ref) are rounded once to fp16 (11 significant bits against
//     bf16's 8, which a single product then meets the accuracy bar with) and handed to the
//     partner wave through LDS;
//   - waves 2p and 2p + 1 form a pair: after a barrier, wave 2p + h accumulates
//     O^T[256 dims x 32 rows] for the pair's rows over value dims [256 h, 256 h + 256) on
//     v_mfma_f32_32x32x16_f16, 16 MFMAs per tile (one per k step and 32-dim block).
// Against a bf16 weight split into a high part and a remainder, this halves the value
// product's matrix work: the issued matrix flops equal the algorithmic ones.
//
// fp16 ranges. A weight is at most 2^kLazy = 2^15 < 65504: a row's reference m_ref is fixed
// by its first valid tile, and a later tile whose maximum exceeds m_ref + kLazy (exp2 units)
// raises it. The wave then scales the row's sum by exp2(m_old - m_new) and posts the factor
// next to its weights; both waves of the pair scale the row's accumulator before they add
// that tile (flag bit kFlagRescaled). bf16 values convert exactly to fp16 between 2^-14 and
// 65504. A worker with a segment that holds a value of magnitude 65504 or more (it would
// overflow), or whose nonzero values all stay below 2^-10 (subnormal fp16 would cost relative
// accuracy), is marked in `redo`, and mla_mfma_kernel<8> recomputes its range in bf16 (flag
// bit kFlagRecomputed).
//
// The tile layout (chunk swizzles, token permutation) is the one in mla_common.h; the fp16
// value buffer has region A's layout.
#include "mla_common.h"

namespace dcp {

namespace pair16 {
constexpr int kWaves = 8;
constexpr int kTile = 32;
constexpr int kRegionB = 32 * 1024;
constexpr int kTileBytes = kRegionB + 32 * 128;  // 36864
constexpr int kRows = kTile / kWaves;            // region-A rows each wave copies per tile
constexpr int kQ0 = 2;                           // of them queued before the scores
constexpr int kOffV = 2 * kTileBytes;            // fp16 value part of the current tile
constexpr int kOffX = kOffV + 32 * 1024;         // weights: 1 KB per wave
constexpr int kOffScale = kOffX + kWaves * 1024; // 128 rescale factors
constexpr int kOffFlag = kOffScale + 128 * 4;    // one word per wave: it raised a reference
constexpr int kLds = kOffFlag + 64;
constexpr float kLazy = 15.f;
constexpr float kF16Max = 65504.f;
constexpr float kF16Small = 0x1p-10f;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
}  // namespace pair16

__global__ void __launch_bounds__(64 * pair16::kWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_pair16_kernel(AttnArgs a, const char* __restrict__ zero_row, int32_t* __restrict__ redo) {
  using namespace pair16;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  char* const v16 = &lds[kOffV];
  char* const xch = &lds[kOffX];
  float* const xscale = (float*)&lds[kOffScale];
  uint32_t* const xflag = (uint32_t*)&lds[kOffFlag];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int hw = wv & 1;          // value dims [256 hw, 256 hw + 256)
  const int pw = wv ^ 1;          // partner wave
  const int n = lane & 15;        // score layout: head within the wave
  const int gq = lane >> 4;       // lane quarter
  const int32_t w = blockIdx.x;
  if (w >= a.P) return;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  const char* __restrict__ Kc = (const char*)a.k;
  const int64_t T_pages = a.pre[a.U];
  const int64_t g0 = worker_begin(T_pages, a.P, w), g1 = worker_begin(T_pages, a.P, w + 1);
  if (g0 >= g1) return;
  int32_t u = find_unit(a.pre, a.U, g0);
  int64_t g = g0;
  int32_t bad = 0, raised = 0, out_of_range = 0;
  const bool bs_pow2 = (a.bs & (a.bs - 1)) == 0;
  const int bs_shift = __builtin_ctz((unsigned)a.bs);

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

    // Block id of the page holding token tile + (lane & 31), read one tile ahead of its use.
    // Token positions fit in 32 bits (max_blocks_per_seq * block_size <= INT32_MAX).
    const int32_t t0i = (int32_t)t0, t1i = (int32_t)t1;
    auto page_of = [&](int32_t tile) -> int32_t {
      int lp = lane;
      asm volatile("" : "+v"(lp));
      const int32_t t = tile + (lp & 31);
      const int32_t tc = t < t1i ? t : t1i - 1;
      return brow[bs_pow2 ? (tc >> bs_shift) : tc / a.bs];
    };
    int32_t blk_next = page_of(t0i);

    // A wave copies region-A rows wv + 8 k (k < 4) and, waves 0-3, the region-B rows
    // 8 wv .. 8 wv + 7 of each tile.
    uint64_t row_src[kRows];
    uint64_t rbase = 0;      // one-page tiles: source of row 0
    uint32_t rstride = 0;    // one-page tiles: bytes between rows (0 for the zero row)
    int32_t rlast = 0;       // one-page tiles: last row before t1 (later rows repeat it)
    int32_t one = 0;         // wave-uniform: the pending tile lies in one page
    uint32_t base_pend = 0;
    auto issue_rows = [&](int k0, int k1) {
      uint32_t lx16 = 16u * (uint32_t)lane;
      asm volatile("" : "+v"(lx16));
      if (one) {
#pragma unroll
        for (int k = k0; k < k1; ++k) {
          const int r = wv + k * kWaves;
          const uint32_t rr = (uint32_t)(r < rlast ? r : rlast);
          dma16s(rbase + (uint64_t)(rr * rstride), lx16 ^ (16u * (uint32_t)mla_swz_a(r)),
                 base_pend + r * 1024);
        }
      } else {
#pragma unroll
        for (int k = k0; k < k1; ++k) {
          const int r = wv + k * kWaves;
          dma16s(row_src[k], lx16 ^ (16u * (uint32_t)mla_swz_a(r)), base_pend + r * 1024);
        }
      }
    };
    auto issue_tile = [&](int32_t tile, int buf, int nrows) -> uint32_t {
      const int32_t blk = blk_next;
      if (tile + kTile < t1i) blk_next = page_of(tile + kTile);
      const uint32_t base = lds_u32(&lds[buf * kTileBytes]);
      base_pend = base;
      one = bs_pow2 ? ((tile >> bs_shift) == ((tile + kTile - 1) >> bs_shift))
                    : (tile / a.bs == (tile + kTile - 1) / a.bs);
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
        const uint32_t m = (uint32_t)__ballot(page_ok && lane < kTile && tile + lane < t1i);
        issue_rows(0, nrows);
        if (wv < 4) {  // region B: four 1 KB blocks of 8 rows
          int lb = lane;
          asm volatile("" : "+v"(lb));
          const int r = 8 * wv + (lb >> 3);
          const uint32_t rr = (uint32_t)(r < rlast ? r : rlast);
          dma16s(rbase, rr * rstride + 1024u + 16u * (uint32_t)((lb & 7) ^ swz_b(r)),
                 base + kRegionB + wv * 1024);
        }
        return m;
      }
      uint64_t rowaddr = (uint64_t)zero_row;
      bool valid = false;
      if (lane < kTile) {
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
      for (int k = 0; k < kRows; ++k) row_src[k] = readlane_u64(rowaddr, wv + k * kWaves);
      issue_rows(0, kRows);
      if (wv < 4) {
        // lane covers row 8 wv + lane / 8: pick its address among the eight rows' addresses
        uint64_t ra = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint64_t aj = readlane_u64(rowaddr, 8 * wv + j);
          ra = ((lane >> 3) == j) ? aj : ra;
        }
        int lb = lane;
        asm volatile("" : "+v"(lb));
        const int r = 8 * wv + (lb >> 3);
        dma16((const char*)ra + 1024 + 16 * ((lb & 7) ^ swz_b(r)),
              base + kRegionB + wv * 1024);
      }
      return mask;
    };

    // This wave's 16 query rows and the last context position they may see.
    int32_t jq = 0;
    const int32_t rho_s = unit_row(a, 0, rg, 16 * wv + n, &jq);
    const int32_t lim = a.Rs == a.Hq ? INT32_MAX
                                  : __builtin_amdgcn_readfirstlane(a.qend[b] + a.j0 + jq);
    bf16x8 qop[kMlaDqk / 32];
    {
      const uint16_t* qrow =
          Q + call_row(a, b, rho_s >= 0 ? rho_s : 0) * kMlaDqk + 8 * gq;
#pragma unroll
      for (int j = 0; j < kMlaDqk / 32; ++j)
        qop[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * j));
    }

    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    float m_ref = kNegInf, l_run = 0.f;
    f16x2 vmax = {(_Float16)0.f, (_Float16)0.f};  // largest value magnitude converted

    uint32_t mask_next = issue_tile(t0i, 0, kRows);
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): the copies of the first tile
    __syncthreads();
    int cur = 0;
    for (int32_t tile = t0i; tile < t1i; tile += kTile) {
      const int32_t dl = lim - tile;
      const uint32_t mask =
          mask_next & (dl < 0 ? 0u : dl >= kTile - 1 ? 0xFFFFFFFFu : (2u << dl) - 1u);
      const bool more = tile + kTile < t1i;
      __builtin_amdgcn_s_setprio(1);
      if (more) mask_next = issue_tile(tile + kTile, cur ^ 1, kQ0);
      __builtin_amdgcn_s_setprio(0);
      const char* tb = &lds[cur * kTileBytes];

      // S^T = K . Q^T for the two 16-row subtiles (chains alternate, K reads kPre ahead)
      int lk = lane;
      asm volatile("" : "+v"(lk));
      const int kr0 = tok_of_row(lk & 15), kq = lk >> 4;
      const int kb = kr0 * 1024, kxq = 16 * (kq ^ mla_swz_a(kr0));
      const int kbB = kRegionB + kr0 * 128, kxBq = 16 * (kq ^ (kr0 & 7));
      auto kread = [&](int idx) -> bf16x8 {  // idx = 2 j + at
        const int at = idx & 1, j = idx >> 1;
        const char* p = (j < 16) ? tb + kb + 16384 * at + ((64 * j) ^ kxq)
                                 : tb + kbB + 2048 * at + ((64 * (j - 16)) ^ kxBq);
        return __builtin_bit_cast(bf16x8, *(const u32x4*)p);
      };
      constexpr int kPre = 4;
      f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 kbuf[kPre];
#pragma unroll
      for (int q = 0; q < kPre; ++q) kbuf[q] = kread(q);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int idx = 0; idx < 2 * (kMlaDqk / 32); ++idx) {
        const bf16x8 kop = kbuf[idx % kPre];
        if (idx + kPre < 2 * (kMlaDqk / 32)) kbuf[idx % kPre] = kread(idx + kPre);
        s[idx & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[idx >> 1], s[idx & 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      __builtin_amdgcn_s_setprio(1);
      if (more && one) issue_rows(kQ0, kRows);  // the rest of a one-page tile's row copies
      __builtin_amdgcn_s_setprio(0);

      // this wave's 4 latent rows of the tile, value dims 0..511, to fp16 (same positions)
      {
        int lc = lane;
        asm volatile("" : "+v"(lc));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int off = (4 * wv + k) * 1024 + 16 * lc;
          const u32x4 x = *(const u32x4*)(tb + off);
          u32x4 y;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f16x2 h = {(_Float16)__uint_as_float(x[q] << 16),
                             (_Float16)__uint_as_float(x[q] & 0xFFFF0000u)};
            vmax = __builtin_elementwise_max(vmax, __builtin_elementwise_abs(h));
            y[q] = __builtin_bit_cast(uint32_t, h);
          }
          *(u32x4*)(v16 + off) = y;
        }
      }

      // weights against the reference; s[at][i] is MFMA row 4gq + i of subtile at. The mask
      // is wave-uniform; a tile with every token visible skips the per-score masking.
      float x[8];
      float tmax = kNegInf;
      const bool full = mask == 0xFFFFFFFFu;
      if (full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          x[k] = s[k >> 2][k & 3] * a.scale_log2;
          tmax = fmaxf(tmax, x[k]);
        }
      } else {
        int lm = lane;
        asm volatile("" : "+v"(lm));
        const int gqm = lm >> 4;
#pragma unroll
        for (int at = 0; at < 2; ++at)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = 16 * at + tok_of_row(4 * gqm + i);
            const float v = ((mask >> tok) & 1u) ? s[at][i] * a.scale_log2 : kNegInf;
            x[4 * at + i] = v;
            tmax = fmaxf(tmax, v);
          }
      }
      tmax = quad_max(tmax);
      // first valid tile of the row (O and l are zero): it fixes the reference; a tile far
      // above it raises the reference, and the row's sum and accumulator are scaled
      float scale = 1.f;
      if (m_ref == kNegInf) {
        m_ref = tmax;
      } else if (tmax > m_ref + kLazy) {
        scale = fast_exp2(m_ref - tmax);
        m_ref = tmax;
      }
      const bool raise_any = __ballot(scale != 1.f) != 0;  // wave-uniform
      float pw8[8];
      if (full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) pw8[k] = fast_exp2(x[k] - m_ref);
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) pw8[k] = (x[k] == kNegInf) ? 0.f : fast_exp2(x[k] - m_ref);
      }
      // fp16 weights packed in pairs
      float psum = 0.f;
      u32x4 hpk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float p0 = pw8[2 * q], p1 = pw8[2 * q + 1];
        psum += p0 + p1;
        const f16x2 h = {(_Float16)p0, (_Float16)p1};
        hpk[q] = __builtin_bit_cast(uint32_t, h);
      }
      l_run = l_run * scale + psum;

      // hand the weights (and any raised rows' factors) to the partner wave
      *(u32x4*)(xch + wv * 1024 + lane * 16) = hpk;
      if (raise_any) {
        raised = 1;
        if (gq == 0) xscale[16 * wv + n] = scale;
      }
      if (lane == 0) xflag[wv] = raise_any ? 1u : 0u;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // O^T[256 dims x 32 rows] += V^T . P over two 16-token k steps; B operand columns
      // 0..15 = own rows, 16..31 = partner rows; k step 0 holds the tokens of lane quarters 0
      // and 2 of the score layout, k step 1 those of quarters 1 and 3
      int lv = lane;
      asm volatile("" : "+v"(lv));
      const int vn = lv & 15, vq = lv >> 4;
      const int vrow0 = 8 * (vq >> 1) + 2 * (vn >> 2);
      const int vb = vrow0 * 1024 + 512 * (hw ^ (vq >> 1)) + 8 * (vn & 1);
      const int vxq = 16 * (((16 * (vq & 1)) | ((vn & 3) >> 1)) ^ (2 * vrow0));
      const int xo = 1024 * ((vq & 1) ? pw : wv) + 16 * (vn + 32 * (vq >> 1));
      const f16x8 ph[2] = {__builtin_bit_cast(f16x8, *(const u32x4*)(xch + xo)),
                           __builtin_bit_cast(f16x8, *(const u32x4*)(xch + xo + 256))};
      // rows whose reference a wave of this pair raised at this tile: accumulator first
      {
        const uint32_t f_own = xflag[wv], f_par = xflag[pw];
        if ((f_own | f_par) != 0u) {
          const int c32 = lane & 31;
          const int hrow = c32 < 16 ? 16 * wv + c32 : 16 * pw + (c32 - 16);
          const uint32_t mine = c32 < 16 ? f_own : f_par;
          const float sc = mine ? xscale[hrow] : 1.f;
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[k][r] *= sc;
        }
      }
      auto vread = [&](int step) -> f16x8 {  // step = 8 s2 + mt
        const int s2 = step >> 3, mt = step & 7;
        const char* v0 = v16 + vb + 1024 * s2 + ((32 * (mt ^ s2)) ^ vxq);
        return __builtin_bit_cast(f16x8, mla_tr_pair(v0, v0 + 16 * 1024));
      };
      __builtin_amdgcn_s_setprio(1);
      constexpr int kVPre = 2;
      f16x8 vbuf[kVPre];
#pragma unroll
      for (int q = 0; q < kVPre; ++q) vbuf[q] = vread(q);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int step = 0; step < 16; ++step) {
        const int s2 = step >> 3, mt = step & 7;
        const f16x8 vop = vbuf[step % kVPre];
        if (step + kVPre < 16) vbuf[step % kVPre] = vread(step + kVPre);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop, ph[s2], acc[mt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): the next tile's copies landed
      __syncthreads();
      cur ^= 1;
    }

    // finalise: every wave is past the last tile's barrier, so the exchange area is free.
    // Besides (l, m) of its rows each wave posts the largest value magnitude it converted.
    {
      const float l_own = quad_sum(l_run);
      float* xf = (float*)xch;
      if (gq == 0) {
        xf[2 * (16 * wv + n)] = l_own;
        xf[2 * (16 * wv + n) + 1] = m_ref;
      }
      float vm = fmaxf((float)vmax[0], (float)vmax[1]);
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) vm = fmaxf(vm, __shfl_xor(vm, off, 64));
      if (lane == 0) xscale[wv] = vm;
      vmax = f16x2{(_Float16)0.f, (_Float16)0.f};
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    {
      float vm = 0.f;
#pragma unroll
      for (int k = 0; k < kWaves; ++k) vm = fmaxf(vm, xscale[k]);
      // a value beyond fp16's range, or a segment whose values are all subnormal-sized
      if (vm >= kF16Max || (vm > 0.f && vm < kF16Small)) out_of_range = 1;
    }
    const int c32 = lane & 31;
    const int hrow = c32 < 16 ? 16 * wv + c32 : 16 * pw + (c32 - 16);  // row within the unit
    const float lc = ((const float*)xch)[2 * hrow];
    const float mc = ((const float*)xch)[2 * hrow + 1];
    int32_t jr = 0;
    const int32_t rho = unit_row(a, 0, rg, hrow, &jr);
    const float inv = lc > 0.f ? 1.f / lc : 0.f;
    float* dst_o;
    float* dst_l;
    if (whole) {
      dst_o = a.part_o + part_row(a, bsi, rho >= 0 ? rho : 0) * kMlaDv;
      dst_l = a.part_lse + part_row(a, bsi, rho >= 0 ? rho : 0);
    } else {
      const int32_t slot = piece_slot(w, first);
      dst_o = a.piece_o + ((int64_t)slot * a.Ru + hrow) * kMlaDv;
      dst_l = a.piece_lse + (int64_t)slot * a.Ru + hrow;
    }
    if (rho >= 0) {
      // acc[mt][4 qd + i] is dim 256 hw + 16 mt + 128 (qd >> 1) + 8 (qd & 1) + 4 (lane >> 5) + i
      const int dbase = 256 * hw + 4 * (lane >> 5);
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
          *(f32x4*)(dst_o + dbase + 16 * mt + 128 * (qd >> 1) + 8 * (qd & 1)) =
              f32x4{acc[mt][4 * qd], acc[mt][4 * qd + 1], acc[mt][4 * qd + 2],
                    acc[mt][4 * qd + 3]} * inv;
      if (lane < 16) *dst_l = lc > 0.f ? (mc + fast_log2(lc)) * kLn2 : kNegInf;
    }
    // the next segment's first weights, flags and factors are written only after every
    // (l, m) and magnitude read
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    g = sg1;
  }
  if (__any(bad) && lane == 0) atomicOr(a.flags, kFlagBadBlock);
  if (__any(raised) && lane == 0) atomicOr(a.flags, kFlagRescaled);
  if (__any(out_of_range) && lane == 0) {
    redo[w] = 1;
    atomicOr(a.flags, kFlagRecomputed);
  }
}

hipError_t launch_mla_pair16(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_pair16_kernel, dim3(a.P), dim3(64 * pair16::kWaves), 0, stream, a,
                     a.zero_row, a.redo);
  return hipGetLastError();
}

}  // namespace dcp
