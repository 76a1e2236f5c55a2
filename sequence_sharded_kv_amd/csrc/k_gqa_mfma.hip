// GQA partial attention with bf16 MFMA, for groups of up to 16 query heads per KV head (the
// dispatcher uses it for head dim 64; head dim 128 goes to the 32-row kernel in k_gqa_chunk.hip).
//
// One wave is one stream-K worker and owns (segment of a (request, shard, kv head) unit) at
// a time. Per 32-token tile:
//   S^T[32 tok x 16 heads] = K[32 x D] . Q^T[D x 16]   v_mfma_f32_16x16x32_bf16, K rows loaded
//                                                     straight from HBM as the A operand,
//                                                     Q of the group held as the B operand;
//   online softmax per head (column of S^T): each lane holds 8 scores of one head, the max
//   and the sums are reduced over the head's four lanes with lane swaps;
//   O^T[D x 16] += V^T[D x 32] . P^T[32 x 16]          V staged row-major in the wave's own
//                                                     LDS tile and read back transposed with
//                                                     ds_read_b64_tr_b16; P from registers.
// P is split into a bf16 high part and a bf16 remainder (two MFMAs) so that the weights
// carry about 16 mantissa bits; rounding P to one bf16 alone would cost ~1e-3 relative error.
// K and V of the next tile sit in a second register set whose loads are queued before the
// current tile is computed (their block ids were read one tile earlier still), so every wave
// keeps a whole tile in flight; at 244 registers two waves share each SIMD.
#include "device_common.h"

namespace dcp {

constexpr int kGqaWaves = 4;     // waves per workgroup (independent workers)
constexpr int kGqaTile = 32;     // tokens per tile

template <int D>
struct GqaCfg {
  static constexpr int kSteps = D / 32;          // MFMA k-steps for Q.K
  static constexpr int kMt = D / 16;             // M tiles of O^T
  static constexpr int kRowBytes = D * 2 + 32;   // padded LDS row of the V tile
  static constexpr int kLdsPerWave = kGqaTile * kRowBytes;
};

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ bf16x8 tr_pair(const char* lo, const char* hi) {
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  i16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, z);
}

// max / sum over the four lanes n, n+16, n+32, n+48 that hold one head, with the VALU lane
// swaps of gfx950 (no LDS round trip)
__device__ __forceinline__ float gqa_quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float gqa_quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The K and V registers of one tile: lane (n, gq) holds, for its tokens tile + n and
// tile + 16 + n, K dims 32 j + 8 gq .. +8 (the MFMA A operand) and V chunks gq, gq + 4, ...
template <int D>
struct GqaTileRegs {
  u32x4 k[2][GqaCfg<D>::kSteps];
  u32x4 v[2][D / 32];
  uint32_t mask;  // bit r: token tile + r is valid
};

template <int D>
__global__ void __launch_bounds__(64 * kGqaWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
gqa_mfma_kernel(AttnArgs a) {
  using C = GqaCfg<D>;
  extern __shared__ char gqa_lds[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;       // head within the group / token row within a subtile
  const int gq = lane >> 4;      // lane quarter
  char* vt = gqa_lds + wv * C::kLdsPerWave;
  const int32_t w = blockIdx.x * kGqaWaves + wv;
  if (w >= a.P) return;
  const uint16_t* __restrict__ Q = (const uint16_t*)a.q;
  const uint16_t* __restrict__ K = (const uint16_t*)a.k;
  const uint16_t* __restrict__ V = (const uint16_t*)a.v;
  const int64_t T_pages = a.pre[a.U];
  const int64_t g0 = worker_begin(T_pages, a.P, w), g1 = worker_begin(T_pages, a.P, w + 1);
  if (g0 >= g1) return;
  const int32_t bs = a.bs;
  const bool bs_pow2 = (bs & (bs - 1)) == 0;
  const int bs_shift = __builtin_ctz((unsigned)bs);
  int32_t u = find_unit(a.pre, a.U, g0);
  int64_t g = g0;
  int32_t bad = 0;

  while (g < g1) {
    while ((int64_t)a.pre[u + 1] <= g) ++u;
    const int64_t up0 = a.pre[u], up1 = a.pre[u + 1];
    const int64_t sg1 = up1 < g1 ? up1 : g1;
    const int32_t per_bs = a.Hkv * a.NRg;
    const int32_t bsi = u / per_bs, hsub = u - bsi * per_bs;
    const int32_t kvh = hsub / a.NRg, rg = hsub - kvh * a.NRg;
    const int32_t b = bsi / a.S;
    const int64_t ta = a.ubounds[2 * bsi], te = a.ubounds[2 * bsi + 1];
    const int64_t pa = ta / bs;
    int64_t t0 = (pa + (g - up0)) * bs, t1 = (pa + (sg1 - up0)) * bs;
    if (t0 < ta) t0 = ta;
    if (t1 > te) t1 = te;
    const bool whole = (g == up0) && (sg1 == up1);
    const bool first = (g == g0);
    const int32_t* brow = a.block_table + (int64_t)b * a.max_blocks;
    // Token positions fit in 32 bits (max_blocks_per_seq * block_size <= INT32_MAX).
    const int32_t t0i = (int32_t)t0, t1i = (int32_t)t1;

    // MFMA column n is query row rho (head of KV head kvh, query token jq), or padding; lim is
    // the last context position the row may see.
    int32_t jq = 0;
    const int32_t rho = unit_row(a, kvh, rg, n, &jq);
    const bool hv = rho >= 0;
    const int32_t lim = a.Rs == a.Hq ? INT32_MAX : a.qend[b] + a.j0 + jq;
    // Q^T as the B operand: lane (n, gq) holds q[rho][32j + 8gq .. +8]
    bf16x8 qop[C::kSteps];
    {
      const uint16_t* qrow = Q + call_row(a, b, hv ? rho : 0) * D;
#pragma unroll
      for (int j = 0; j < C::kSteps; ++j) {
        u32x4 raw = *(const u32x4*)(qrow + 32 * j + 8 * gq);
        if (!hv) raw = u32x4{0, 0, 0, 0};
        qop[j] = __builtin_bit_cast(bf16x8, raw);
      }
    }

    auto page_idx = [&](int32_t t) -> int32_t { return bs_pow2 ? (t >> bs_shift) : t / bs; };
    auto slot_of = [&](int32_t t) -> int32_t { return bs_pow2 ? (t & (bs - 1)) : t % bs; };
    // block ids of this lane's two tokens of a tile (clamped into the segment)
    auto pages_of = [&](int32_t tile, int32_t* pg) {
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        int32_t t = tile + 16 * at + n;
        if (t >= t1i) t = t1i - 1;
        pg[at] = brow[page_idx(t)];
      }
    };
    // queue the loads of tile `tile` whose tokens' block ids are pg
    auto load_tile = [&](int32_t tile, const int32_t* pg, GqaTileRegs<D>& r) {
      uint32_t m = 0;
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        int32_t t = tile + 16 * at + n;
        const bool in = t < t1i;
        if (!in) t = t1i - 1;
        const int32_t blk = pg[at];
        const bool page_ok = blk >= 0 && blk < a.num_blocks;
        bad |= (in && !page_ok) ? 1 : 0;
        const uint64_t bal = __ballot(in && page_ok);
        m |= (uint32_t)(bal & 0xFFFF) << (16 * at);
        // row index (block, kv head, slot) of the token; a token of an invalid page reads the
        // workspace's zero row and is masked out
        const uint32_t row = ((uint32_t)blk * (uint32_t)a.Hkv + (uint32_t)kvh) * (uint32_t)bs +
                             (uint32_t)slot_of(t);
        const uint16_t* kp = page_ok ? K + (uint64_t)row * D : (const uint16_t*)a.zero_row;
        const uint16_t* vp = page_ok ? V + (uint64_t)row * D : (const uint16_t*)a.zero_row;
#pragma unroll
        for (int j = 0; j < C::kSteps; ++j) r.k[at][j] = *(const u32x4*)(kp + 32 * j + 8 * gq);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) r.v[at][i] = *(const u32x4*)(vp + 8 * (4 * i + gq));
      }
      r.mask = m;
    };

    f32x4 acc[C::kMt];
#pragma unroll
    for (int i = 0; i < C::kMt; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    // One tile: stage V of `cur` in LDS, queue the loads of the next tile into `nxt` (its
    // block ids were read one tile earlier), read the block ids of the tile after it, then
    // scores, softmax and P.V of `cur`.
    int32_t pg_next[2], pg_after[2];
    auto step = [&](int32_t tile, GqaTileRegs<D>& cur, GqaTileRegs<D>& nxt) {
#pragma unroll
      for (int at = 0; at < 2; ++at)
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          *(u32x4*)(vt + (16 * at + n) * C::kRowBytes + (4 * i + gq) * 16) = cur.v[at][i];
      if (tile + kGqaTile < t1i) {
        load_tile(tile + kGqaTile, pg_next, nxt);
        if (tile + 2 * kGqaTile < t1i) {
          pages_of(tile + 2 * kGqaTile, pg_after);
          pg_next[0] = pg_after[0];
          pg_next[1] = pg_after[1];
        }
      }
      // S^T = K . Q^T
      f32x4 s[2];
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        s[at] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < C::kSteps; ++j)
          s[at] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.k[at][j]),
                                                          qop[j], s[at], 0, 0, 0);
      }
      // online softmax: lane holds tokens 16at + 4gq + i of row n (its valid tokens up to lim)
      const int32_t dl = lim - tile;
      const uint32_t mask =
          cur.mask & (dl < 0 ? 0u : dl >= kGqaTile - 1 ? 0xFFFFFFFFu : (2u << dl) - 1u);
      float x[8];
      float tmax = kNegInf;
#pragma unroll
      for (int at = 0; at < 2; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 16 * at + 4 * gq + i;
          const float v = ((mask >> tok) & 1u) ? s[at][i] * a.scale_log2 : kNegInf;
          x[4 * at + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = gqa_quad_max(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      float psum = 0.f;
      bf16x8 phi, plo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float p = (x[k] == kNegInf) ? 0.f : fast_exp2(x[k] - m_new);
        psum += p;
        const __bf16 h = (__bf16)p;
        phi[k] = h;
        plo[k] = (__bf16)(p - (float)h);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int i = 0; i < C::kMt; ++i) acc[i] *= alpha;
      }
      // O^T += V^T . P^T ; A operand rows: tokens 4gq + e (slots 0..3), 16 + 4gq + e (4..7)
      const char* rlo = vt + (4 * gq + (n >> 2)) * C::kRowBytes + (n & 3) * 8;
      const char* rhi = rlo + 16 * C::kRowBytes;
#pragma unroll
      for (int mt = 0; mt < C::kMt; ++mt) {
        const bf16x8 vop = tr_pair(rlo + mt * 32, rhi + mt * 32);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, acc[mt], 0, 0, 0);
      }
    };

    GqaTileRegs<D> ra, rb;
    {
      int32_t pg0[2];
      pages_of(t0i, pg0);
      load_tile(t0i, pg0, ra);
      if (t0i + kGqaTile < t1i) pages_of(t0i + kGqaTile, pg_next);
    }
    for (int32_t tile = t0i; tile < t1i; tile += 2 * kGqaTile) {
      step(tile, ra, rb);
      if (tile + kGqaTile < t1i) step(tile + kGqaTile, rb, ra);
    }

    // finalise: l over the four lanes of head n
    const float l = gqa_quad_sum(l_run);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst_o;
    float* dst_l;
    if (whole) {
      dst_o = a.part_o + part_row(a, bsi, rho) * D;
      dst_l = a.part_lse + part_row(a, bsi, rho);
    } else {
      int32_t slot = piece_slot(w, first);
      dst_o = a.piece_o + ((int64_t)slot * a.Ru + n) * D;
      dst_l = a.piece_lse + (int64_t)slot * a.Ru + n;
    }
    if (hv) {
#pragma unroll
      for (int mt = 0; mt < C::kMt; ++mt) *(f32x4*)(dst_o + 16 * mt + 4 * gq) = acc[mt] * inv;
      if (gq == 0) *dst_l = l > 0.f ? (m_run + fast_log2(l)) * kLn2 : kNegInf;
    }
    g = sg1;
  }
  if (bad) atomicOr(a.flags, kFlagBadBlock);
}

int32_t gqa_mfma_workers(int device, int32_t Dqk, int32_t max_workers) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int per_cu = 2;  // workgroups resident per CU
  int32_t p = cus * kGqaWaves * per_cu;
  (void)Dqk;
  return p < max_workers ? p : max_workers;
}

template <int D>
static hipError_t launch_gqa_t(const AttnArgs& a, hipStream_t stream) {
  size_t lds = (size_t)kGqaWaves * GqaCfg<D>::kLdsPerWave;
  int32_t grid = (a.P + kGqaWaves - 1) / kGqaWaves;
  hipLaunchKernelGGL((gqa_mfma_kernel<D>), dim3(grid), dim3(64 * kGqaWaves), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_gqa_mfma(const AttnArgs& a, hipStream_t stream) {
  switch (a.Dqk) {
    case 64: return launch_gqa_t<64>(a, stream);
    case 128: return launch_gqa_t<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dcp
