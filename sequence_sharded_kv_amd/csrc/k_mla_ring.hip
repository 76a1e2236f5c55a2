// MLA partial attention for units of 64 query rows (64 heads of one decode token, or 32 heads
// x 2 tokens, 16 x 3-4): one workgroup of 12 waves per CU with a ring of LDS tiles and waves
// specialised by role, so that the copies, the scores and the value product of consecutive
// tiles proceed side by side.
//
// Per 32-token tile (36 KB: 32 latent rows of 1152 B):
//   - copy waves 8-11 queue the tile's 36 HBM -> LDS copies (global_load_lds_dwordx4, 1 KB
//     each; 8 latent rows and one 1 KB block of rope rows per wave) two tiles ahead of its
//     scores, read the page ids through the scalar cache, and publish the tile's valid-token
//     mask. A wave queues copies at about one per 90 cycles here, and stalls while the memory
//     pipeline is full: one wave alone could not keep 36 KB per tile in flight, and the
//     compute waves never wait on a copy's issue;
//   - score waves 0-3 (head block hb = wave, 16 rows each) compute
//     S^T[32 tokens x 16 heads] = K[32 x 576] . Q^T[576 x 16] on v_mfma_f32_16x16x32_bf16
//     (2 subtiles x 18 k steps; K from LDS, the block's Q slice resident in registers), the
//     weights p = exp2(s - m_ref) in fp32, split into a bf16 high part and a bf16 remainder,
//     and write them to an 8 KB exchange buffer;
//   - value waves 4-7 (row half rh = w & 1, value half hw = (w >> 1) & 1) accumulate
//     O^T[256 dims x 32 rows] += V^T[256 x 32 tokens] . P^T[32 tokens x 32 rows] on
//     v_mfma_f32_32x32x16_bf16 (2 k steps x 8 blocks x 2 parts = 32 MFMAs; V = the first 512
//     dims of the same LDS rows, read transposed with ds_read_b64_tr_b16).
// Iteration i scores tile i while the value waves multiply tile i - 1 and the copies of tile
// i + 2 are queued; one workgroup barrier per iteration. A SIMD holds one score wave (36 MFMAs
// and the softmax) beside one value wave (32 MFMAs). The latent dims 0..511 of a tile (32 KB)
// live in a four-slot ring, since the value product reads them one iteration after the scores;
// the rope dims 512..575 (4 KB) in a three-slot ring; the exchange is double-buffered.
// The tile layout (chunk swizzles, token permutation) is the one in mla_common.h.
//
// Reference max: a row's weights are exp2(s - m_ref) with m_ref fixed by the first tile in
// which the row has a valid token (its weights and sum are still zero then), so the value
// accumulator is not rescaled tile by tile. Only a later tile whose maximum exceeds
// m_ref + kLazy (exp2 units; the weights stay below 2^kLazy otherwise) raises the row's
// reference to that maximum: the score wave scales the row's sum by exp2(m_old - m_new) and
// posts the factor with the tile's weights, and the value waves scale the row's accumulator
// by it before they add that tile. Flag bit kFlagRescaled reports that it happened.
//
// Waits: a copy wave awaits its copies of a tile with a partial vmcnt (the next tile's copies
// stay in flight). Tiles that span pages (block sizes below 32, or ranges not aligned to 32
// tokens) look up one page per row with a vector load, whose wait drains that wave's queue:
// correct, and slower.
#include "mla_common.h"

namespace dcp {

namespace ring {
constexpr int kTile = 32;
constexpr int kSlotsA = 4;                        // dims 0..511: 32 rows x 1 KB
constexpr int kSlotsB = 3;                        // dims 512..575: 32 rows x 128 B
constexpr int kBytesA = 32 * 1024;
constexpr int kBytesB = 32 * 128;
constexpr int kOffB = kSlotsA * kBytesA;          // 131072
// exchange of one tile: the weights (4 score waves x 2 KB), each row's rescale factor, and one
// word per score wave telling whether it raised a reference in this tile
constexpr int kXScale = 4 * 2048;                 // 64 floats
constexpr int kXFlag = kXScale + 64 * 4;          // 4 words
constexpr int kXBytes = kXFlag + 64;              // 8512
constexpr int kOffX = kOffB + kSlotsB * kBytesB;  // 143360
constexpr int kOffMask = kOffX + 2 * kXBytes;     // 160384: valid-token mask per A slot
constexpr int kLds = kOffMask + 64;               // 160448 B of the 160 KB
constexpr int kCopyWave0 = 8;                     // waves 8..11 copy
constexpr int kWaves = 12;
constexpr float kLazy = 64.f;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((address_space(4))) const int32_t cint32_t;
}  // namespace ring

__global__ void __launch_bounds__(64 * ring::kWaves)
mla_ring_kernel(AttnArgs a, const char* __restrict__ zero_row) {
  using namespace ring;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  char* const xch = &lds[kOffX];  // two exchange buffers, tile i in buffer i & 1
  uint32_t* const lmask = (uint32_t*)&lds[kOffMask];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const bool copier = wv >= kCopyWave0;
  const int cw = wv & 3;                      // copy waves: latent rows cw + 4 j, rope block cw
  const bool scorer = wv < 4;
  const int hb = wv & 3;                      // score waves: rows 16 hb .. 16 hb + 15
  const int rh = wv & 1, hw = (wv >> 1) & 1;  // value waves: rows 32 rh.., dims 256 hw..
  const int n = lane & 15;                    // score layout: head within the block
  const int gq = lane >> 4;                   // lane quarter
  const int32_t w = blockIdx.x;
  if (w >= a.P) return;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  const char* __restrict__ Kc = (const char*)a.k;
  const int64_t T_pages = a.pre[a.U];
  const int64_t g0 = worker_begin(T_pages, a.P, w), g1 = worker_begin(T_pages, a.P, w + 1);
  if (g0 >= g1) return;
  int32_t u = find_unit(a.pre, a.U, g0);
  int64_t g = g0;
  int32_t bad = 0, raised = 0;
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
    // token positions fit in 32 bits (max_blocks_per_seq * block_size <= INT32_MAX)
    const int32_t t0i = (int32_t)t0, t1i = (int32_t)t1;
    const int32_t ntile = t1i > t0i ? (t1i - t0i + kTile - 1) / kTile : 0;

    if (copier) {
      // ------------------------------------------------------------ copy wave
      const int32_t* brow = a.block_table + (int64_t)b * a.max_blocks;
      auto spage = [&](int32_t t) -> int32_t {  // page of token t (< t1), scalar cache
        return ((cint32_t*)brow)[bs_pow2 ? (t >> bs_shift) : t / a.bs];
      };
      // Queue this wave's 9 copies of tile k of the segment (region-A rows cw + 4 j into A
      // slot k % 4, the region-B block of rows 8 cw .. 8 cw + 7 into B slot k % 3) and store
      // the tile's valid-token mask. `pg` is the page of the tile's first token, used when the
      // tile lies in one page.
      auto issue = [&](int32_t k, int32_t pg) {
        const int32_t tile = t0i + kTile * k;
        const uint32_t baseA = lds_u32(&lds[(k & (kSlotsA - 1)) * kBytesA]);
        const uint32_t baseB = lds_u32(&lds[kOffB + (k % kSlotsB) * kBytesB]);
        const bool one = bs_pow2 ? ((tile >> bs_shift) == ((tile + kTile - 1) >> bs_shift))
                                 : (tile / a.bs == (tile + kTile - 1) / a.bs);
        const int32_t rlast = t1i - 1 - tile;  // last row before t1 (later rows repeat it)
        uint32_t lx16 = 16u * (uint32_t)lane;
        asm volatile("" : "+v"(lx16));
        uint32_t mask;
        if (one) {
          // rows past t1 repeat the last valid row: the page's later slots may hold anything,
          // and a NaN there would survive its zero weight in the value product
          const bool page_ok = pg >= 0 && pg < a.num_blocks;
          const uint32_t slot0 = bs_pow2 ? (uint32_t)(tile & (a.bs - 1)) : (uint32_t)(tile % a.bs);
          const uint64_t rbase =
              page_ok ? (uint64_t)Kc + ((uint64_t)(uint32_t)pg * (uint32_t)a.bs + slot0) *
                                           (kMlaDqk * 2)
                      : (uint64_t)zero_row;
          const uint32_t rstride = page_ok ? kMlaDqk * 2 : 0;
          if (!page_ok) bad = 1;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = cw + 4 * j;
            const uint32_t rr = (uint32_t)(r < rlast ? r : rlast);
            dma16s(rbase + (uint64_t)(rr * rstride), lx16 ^ (16u * (uint32_t)mla_swz_a(r)),
                   baseA + r * 1024);
          }
          int lb = lane;
          asm volatile("" : "+v"(lb));
          const int r = 8 * cw + (lb >> 3);
          const uint32_t rr = (uint32_t)(r < rlast ? r : rlast);
          dma16s(rbase, rr * rstride + 1024u + 16u * (uint32_t)((lb & 7) ^ swz_b(r)),
                 baseB + cw * 1024);
          const int32_t nv = t1i - tile;  // >= 1
          mask = page_ok ? (nv >= kTile ? 0xFFFFFFFFu : (1u << nv) - 1u) : 0u;
        } else {
          // the tile spans pages: lane r < 32 looks up row r's page
          uint64_t rowaddr = (uint64_t)zero_row;
          bool valid = false;
          if (lane < kTile) {
            const int32_t t = tile + lane;
            const int32_t tc = t < t1i ? t : t1i - 1;
            const int32_t blk = brow[bs_pow2 ? (tc >> bs_shift) : tc / a.bs];
            const bool page_ok = blk >= 0 && blk < a.num_blocks;
            // row index < num_blocks * block_size rows of 1152 B: below 2^31 for any pool
            // that fits in device memory
            const uint32_t slot = bs_pow2 ? (uint32_t)(tc & (a.bs - 1)) : (uint32_t)(tc % a.bs);
            const uint32_t row = (uint32_t)blk * (uint32_t)a.bs + slot;
            if (page_ok)
              rowaddr = (uint64_t)Kc + (uint64_t)row * (kMlaDqk * 2);
            else
              bad = 1;
            valid = page_ok && t < t1i;
          }
          mask = (uint32_t)__ballot(valid);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int r = cw + 4 * j;
            dma16s(readlane_u64(rowaddr, r), lx16 ^ (16u * (uint32_t)mla_swz_a(r)),
                   baseA + r * 1024);
          }
          // lane covers row 8 cw + lane / 8: pick its address among the eight rows'
          uint64_t ra = 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint64_t aj = readlane_u64(rowaddr, 8 * cw + j);
            ra = ((lane >> 3) == j) ? aj : ra;
          }
          int lb = lane;
          asm volatile("" : "+v"(lb));
          const int r = 8 * cw + (lb >> 3);
          dma16((const char*)ra + 1024 + 16 * ((lb & 7) ^ swz_b(r)), baseB + cw * 1024);
        }
        if (cw == 0 && lane == 0) lmask[k & (kSlotsA - 1)] = mask;
      };
      // vmcnt(n) with n = 0 or this wave's copies of one tile (the immediate must be a constant)
      auto wait_tile = [&](bool keep_one) {
        if (keep_one)
          __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9): expcnt/lgkmcnt left open
        else
          __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      };
      // prologue: tiles 0 and 1; tile 0 landed before the first barrier
      for (int32_t k = 0; k < 2 && k < ntile; ++k) issue(k, spage(t0i + kTile * k));
      int32_t pg_next = 2 < ntile ? spage(t0i + 2 * kTile) : 0;
      if (ntile > 0) wait_tile(ntile > 1);
      for (int32_t i = 0; i <= ntile; ++i) {
        // the barrier publishes tile i and its mask, and frees the A slot of tile i - 2 and
        // the B slot of tile i - 1
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (i + 2 < ntile) {
          issue(i + 2, pg_next);
          pg_next = i + 3 < ntile ? spage(t0i + kTile * (i + 3)) : 0;
        }
        // tile i + 1 lands before the next barrier; tile i + 2 may stay in flight
        if (i + 1 < ntile) wait_tile(i + 2 < ntile);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // finalise barrier
    } else if (scorer) {
      // ------------------------------------------------------------ score waves
      // 16 query rows (head block hb; one query token per block since 16 | Hq) and the last
      // context position they may see; the Q slice as the MFMA B operand
      int32_t jq = 0;
      const int32_t rho_s = unit_row(a, 0, rg, 16 * hb + n, &jq);
      const int32_t lim = a.Rs == a.Hq ? INT32_MAX
                                    : __builtin_amdgcn_readfirstlane(a.qend[b] + a.j0 + jq);
      bf16x8 qop[kMlaDqk / 32];
      {
        const uint16_t* qrow =
            Q + call_row(a, b, rho_s >= 0 ? rho_s : 0) * kMlaDqk + 8 * gq;
#pragma unroll
        for (int j = 0; j < kMlaDqk / 32; ++j)
          qop[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 32 * j));
        // Q's loads complete here rather than at their first use inside the loop
#pragma unroll
        for (int j = 0; j < kMlaDqk / 32; ++j) asm volatile("" ::"v"(qop[j]));
      }
      float m_ref = kNegInf, l_run = 0.f;
      for (int32_t i = 0; i <= ntile; ++i) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (i < ntile) {
          const int32_t tile = t0i + kTile * i;
          const int32_t dl = lim - tile;
          const uint32_t mask = lmask[i & (kSlotsA - 1)] &
                                (dl < 0 ? 0u : dl >= kTile - 1 ? 0xFFFFFFFFu : (2u << dl) - 1u);
          const char* tA = &lds[(i & (kSlotsA - 1)) * kBytesA];
          const char* tB = &lds[kOffB + (i % kSlotsB) * kBytesB];
          // S^T = K . Q^T for the two 16-row subtiles; the subtiles' chains alternate and the
          // K reads run four ahead
          int lk = lane;
          asm volatile("" : "+v"(lk));
          const int kr0 = tok_of_row(lk & 15), kq = lk >> 4;
          const int kb = kr0 * 1024, kxq = 16 * (kq ^ mla_swz_a(kr0));
          const int kbB = kr0 * 128, kxBq = 16 * (kq ^ (kr0 & 7));
          auto kread = [&](int idx) -> bf16x8 {  // idx = 2 j + at
            const int at = idx & 1, j = idx >> 1;
            const char* p = (j < 16) ? tA + kb + 16384 * at + ((64 * j) ^ kxq)
                                     : tB + kbB + 2048 * at + ((64 * (j - 16)) ^ kxBq);
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
            s[idx & 1] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[idx >> 1], s[idx & 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
          // weights against the reference; s[at][e] is MFMA row 4 gq + e of subtile at. The
          // mask is wave-uniform; a tile with every token visible skips the masking.
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
              for (int e = 0; e < 4; ++e) {
                const int tok = 16 * at + tok_of_row(4 * gqm + e);
                const float v = ((mask >> tok) & 1u) ? s[at][e] * a.scale_log2 : kNegInf;
                x[4 * at + e] = v;
                tmax = fmaxf(tmax, v);
              }
          }
          tmax = quad_max(tmax);
          // first valid tile of the row (O and l are zero): it fixes the reference; a tile
          // far above it raises the reference, and the row's sum and accumulator are scaled
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
          // bf16 high parts packed in pairs, the remainders from the unpacked highs
          float psum = 0.f;
          u32x4 hpk, lpk;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float p0 = pw8[2 * q], p1 = pw8[2 * q + 1];
            psum += p0 + p1;
            typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
            const bf16x2 h = {(__bf16)p0, (__bf16)p1};
            const uint32_t hbits = __builtin_bit_cast(uint32_t, h);
            const float r0 = p0 - __uint_as_float(hbits << 16);
            const float r1 = p1 - __uint_as_float(hbits & 0xFFFF0000u);
            const bf16x2 l = {(__bf16)r0, (__bf16)r1};
            hpk[q] = hbits;
            lpk[q] = __builtin_bit_cast(uint32_t, l);
          }
          l_run = l_run * scale + psum;
          char* xt = xch + (i & 1) * kXBytes;
          char* xb = xt + hb * 2048;
          *(u32x4*)(xb + lane * 16) = hpk;
          *(u32x4*)(xb + 1024 + lane * 16) = lpk;
          if (raise_any) {
            raised = 1;
            if (gq == 0) ((float*)(xt + kXScale))[16 * hb + n] = scale;
          }
          if (lane == 0) ((uint32_t*)(xt + kXFlag))[hb] = raise_any ? 1u : 0u;
        } else {
          // after the last tile: the rows' (l, m) go to the exchange buffer that the last
          // iteration does not read
          const float l_own = quad_sum(l_run);
          float* xf = (float*)(xch + (i & 1) * kXBytes);
          if (gq == 0) {
            xf[2 * (16 * hb + n)] = l_own;
            xf[2 * (16 * hb + n) + 1] = m_ref;
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // finalise barrier
    } else {
      // ------------------------------------------------------------ value waves
      f32x16 acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
      for (int32_t i = 0; i <= ntile; ++i) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (i == 0) continue;
        // O^T[256 dims x 32 rows] += V^T . P over two 16-token k steps of tile i - 1. B
        // operand columns 0..15 are score block 2 rh, 16..31 block 2 rh + 1; k step 0 holds
        // the tokens of score-lane quarters 0 and 2, k step 1 those of quarters 1 and 3.
        const char* tA = &lds[((i - 1) & (kSlotsA - 1)) * kBytesA];
        const char* xb = xch + ((i - 1) & 1) * kXBytes;
        int lv = lane;
        asm volatile("" : "+v"(lv));
        const int vn = lv & 15, vq = lv >> 4;
        const int vrow0 = 8 * (vq >> 1) + 2 * (vn >> 2);
        const int vb = vrow0 * 1024 + 512 * (hw ^ (vq >> 1)) + 8 * (vn & 1);
        const int vxq = 16 * (((16 * (vq & 1)) | ((vn & 3) >> 1)) ^ (2 * vrow0));
        const char* xp = xb + 2048 * (2 * rh + (vq & 1)) + 16 * (vn + 32 * (vq >> 1));
        bf16x8 ph = __builtin_bit_cast(bf16x8, *(const u32x4*)xp);
        bf16x8 pl = __builtin_bit_cast(bf16x8, *(const u32x4*)(xp + 1024));
        // score waves 2 rh and 2 rh + 1 hold this wave's rows: if either raised a reference
        // at tile i - 1, the rows' accumulators are scaled before that tile is added
        typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
        const u32x2 rfl = *(const u32x2*)(xb + kXFlag + 8 * rh);
        if ((rfl[0] | rfl[1]) != 0u) {
          const int hrow = 32 * rh + (lane & 31);
          const uint32_t mine = (lane & 31) < 16 ? rfl[0] : rfl[1];
          const float sc = mine ? ((const float*)(xb + kXScale))[hrow] : 1.f;
#pragma unroll
          for (int k = 0; k < 8; ++k)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[k][r] *= sc;
        }
        auto vread = [&](int step) -> bf16x8 {  // step = 8 s2 + mt
          const int s2 = step >> 3, mt = step & 7;
          const char* v0 = tA + vb + 1024 * s2 + ((32 * (mt ^ s2)) ^ vxq);
          return mla_tr_pair(v0, v0 + 16 * 1024);
        };
        constexpr int kVPre = 2;
        bf16x8 vbuf[kVPre];
#pragma unroll
        for (int q = 0; q < kVPre; ++q) vbuf[q] = vread(q);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int step = 0; step < 16; ++step) {
          const int mt = step & 7;
          const bf16x8 vop = vbuf[step % kVPre];
          if (step + kVPre < 16) vbuf[step % kVPre] = vread(step + kVPre);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, ph, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pl, acc[mt], 0, 0, 0);
          if (step == 7) {  // weights of k step 1
            ph = __builtin_bit_cast(bf16x8, *(const u32x4*)(xp + 256));
            pl = __builtin_bit_cast(bf16x8, *(const u32x4*)(xp + 1280));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // finalise: (l, m) of the rows are in exchange buffer ntile & 1
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      const int hrow = 32 * rh + (lane & 31);  // row within the unit
      const float* xf = (const float*)(xch + (ntile & 1) * kXBytes);
      const float lc = xf[2 * hrow];
      const float mc = xf[2 * hrow + 1];
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
        // acc[mt][4 qd + e] is dim 256 hw + 16 mt + 128 (qd >> 1) + 8 (qd & 1) + 4 (lane >> 5) + e
        const int dbase = 256 * hw + 4 * (lane >> 5);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int qd = 0; qd < 4; ++qd)
            *(f32x4*)(dst_o + dbase + 16 * mt + 128 * (qd >> 1) + 8 * (qd & 1)) =
                f32x4{acc[mt][4 * qd], acc[mt][4 * qd + 1], acc[mt][4 * qd + 2],
                      acc[mt][4 * qd + 3]} * inv;
        if (hw == 0 && lane < 32) *dst_l = lc > 0.f ? (mc + fast_log2(lc)) * kLn2 : kNegInf;
      }
    }
    // the next segment's first weights and masks are written only after every (l, m) read
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    g = sg1;
  }
  if (__any(bad) && lane == 0) atomicOr(a.flags, kFlagBadBlock);
  if (__any(raised) && lane == 0) atomicOr(a.flags, kFlagRescaled);
}

hipError_t launch_mla_ring(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_ring_kernel, dim3(a.P), dim3(64 * ring::kWaves), 0, stream, a,
                     a.zero_row);
  return hipGetLastError();
}

}  // namespace dcp
