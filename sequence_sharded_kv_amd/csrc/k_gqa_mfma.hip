// GQA partial attention with bf16 MFMA, for groups of up to 16 query heads per KV head.
//
// One wave is one stream-K worker and owns (segment of a (request, shard, kv head) unit) at
// a time. Per 32-token tile:
//   S^T[32 tok x 16 heads] = K[32 x D] . Q^T[D x 16]   v_mfma_f32_16x16x32_bf16, K rows loaded
//                                                     straight from HBM as the A operand,
//                                                     Q of the group held as the B operand;
//   online softmax per head (column of S^T): each lane holds 8 scores of one head, the max
//   and the sums need two cross-lane shuffles;
//   O^T[D x 16] += V^T[D x 32] . P^T[32 x 16]          V staged row-major in the wave's own
//                                                     LDS tile and read back transposed with
//                                                     ds_read_b64_tr_b16; P from registers.
// P is split into a bf16 high part and a bf16 remainder (two MFMAs) so that the weights
// carry about 16 mantissa bits; rounding P to one bf16 alone would cost ~1e-3 relative error.
// The next tile's K and V loads are issued before the current tile is computed.
#include "device_common.h"

namespace dcp {

constexpr int kGqaWaves = 4;     // waves per workgroup (independent workers)
constexpr int kGqaTile = 32;     // tokens per tile

template <int D>
struct GqaCfg {
  static constexpr int kSteps = D / 32;          // MFMA k-steps for Q.K
  static constexpr int kMt = D / 16;             // M tiles of O^T
  static constexpr int kRowBytes = D * 2 + 32;   // padded LDS row of the V tile
  static constexpr int kVChunks = kGqaTile * D * 2 / 16 / 64;  // 16-byte V chunks per lane
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

template <int D>
__global__ void __launch_bounds__(64 * kGqaWaves)
gqa_mfma_kernel(AttnArgs a) {
  using C = GqaCfg<D>;
  extern __shared__ char gqa_lds[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n = lane & 15;       // head within the group / token row within an M tile
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
  const int G = a.G;
  int32_t u = find_unit(a.pre, a.U, g0);
  int64_t g = g0;
  int32_t bad = 0;

  while (g < g1) {
    while ((int64_t)a.pre[u + 1] <= g) ++u;
    const int64_t up0 = a.pre[u], up1 = a.pre[u + 1];
    const int64_t sg1 = up1 < g1 ? up1 : g1;
    const int32_t bsi = u / a.Hkv, kvh = u % a.Hkv;
    const int32_t b = bsi / a.S;
    const int64_t ta = a.ubounds[2 * bsi], te = a.ubounds[2 * bsi + 1];
    const int64_t pa = ta / a.bs;
    int64_t t0 = (pa + (g - up0)) * a.bs, t1 = (pa + (sg1 - up0)) * a.bs;
    if (t0 < ta) t0 = ta;
    if (t1 > te) t1 = te;
    const bool whole = (g == up0) && (sg1 == up1);
    const bool first = (g == g0);
    const int32_t* brow = a.block_table + (int64_t)b * a.max_blocks;

    // Q^T as the B operand: lane (n, gq) holds q[n][32j + 8gq .. +8]
    bf16x8 qop[C::kSteps];
    {
      const bool hv = n < G;
      const uint16_t* qrow = Q + ((int64_t)b * a.Hq + kvh * G + (hv ? n : 0)) * D;
#pragma unroll
      for (int j = 0; j < C::kSteps; ++j) {
        u32x4 raw = *(const u32x4*)(qrow + 32 * j + 8 * gq);
        if (!hv) raw = u32x4{0, 0, 0, 0};
        qop[j] = __builtin_bit_cast(bf16x8, raw);
      }
    }

    // row address of token t of this unit (clamped into the segment; invalid pages -> -1)
    auto row_of = [&](int64_t t) -> int64_t {
      if (t >= t1) t = t1 - 1;
      int32_t blk = brow[t / a.bs];
      if (blk < 0 || blk >= a.num_blocks) return -1;
      return (((int64_t)blk * a.Hkv + kvh) * a.bs + t % a.bs) * D;
    };

    u32x4 kreg[2][C::kSteps];
    u32x4 vreg[C::kVChunks];
    uint32_t vmask = 0;  // bit r: token tile+r is valid
    auto load_tile = [&](int64_t tile) {
      // K: lane loads token tile + 16a + n, dims 32j + 8gq
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        int64_t t = tile + 16 * at + n;
        int64_t r = row_of(t);
        bool ok = (t < t1) && (r >= 0);
        uint64_t bal = __ballot(ok);
        if (at == 0) vmask = (uint32_t)(bal & 0xFFFF); else vmask |= (uint32_t)(bal & 0xFFFF) << 16;
        if (r < 0) { bad |= (t < t1); r = 0; }
        const uint16_t* kp = K + r;
#pragma unroll
        for (int j = 0; j < C::kSteps; ++j) kreg[at][j] = *(const u32x4*)(kp + 32 * j + 8 * gq);
      }
      // V: chunk c = lane + 64i covers token c / (D/8), dims 8 (c % (D/8))
#pragma unroll
      for (int i = 0; i < C::kVChunks; ++i) {
        int c = lane + 64 * i;
        int tr = c / (D / 8), col = c % (D / 8);
        int64_t r = row_of(tile + tr);
        u32x4 x = {0, 0, 0, 0};
        if (r >= 0) x = *(const u32x4*)(V + r + 8 * col);
        vreg[i] = x;
      }
    };

    f32x4 acc[C::kMt];
#pragma unroll
    for (int i = 0; i < C::kMt; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    load_tile(t0);
    for (int64_t tile = t0; tile < t1; tile += kGqaTile) {
      u32x4 kcur[2][C::kSteps];
#pragma unroll
      for (int at = 0; at < 2; ++at)
#pragma unroll
        for (int j = 0; j < C::kSteps; ++j) kcur[at][j] = kreg[at][j];
      const uint32_t mask = vmask;
      // stage V of this tile into the wave's LDS tile
#pragma unroll
      for (int i = 0; i < C::kVChunks; ++i) {
        int c = lane + 64 * i;
        int tr = c / (D / 8), col = c % (D / 8);
        *(u32x4*)(vt + tr * C::kRowBytes + col * 16) = vreg[i];
      }
      if (tile + kGqaTile < t1) load_tile(tile + kGqaTile);

      // S^T = K . Q^T
      f32x4 s[2];
#pragma unroll
      for (int at = 0; at < 2; ++at) {
        s[at] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < C::kSteps; ++j)
          s[at] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kcur[at][j]),
                                                          qop[j], s[at], 0, 0, 0);
      }
      // online softmax: lane holds tokens 16at + 4gq + i of head n
      float x[8];
      float tmax = kNegInf;
#pragma unroll
      for (int at = 0; at < 2; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int tok = 16 * at + 4 * gq + i;
          float v = ((mask >> tok) & 1u) ? s[at][i] * a.scale_log2 : kNegInf;
          x[4 * at + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      float psum = 0.f;
      bf16x8 phi, plo;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float p = (x[k] == kNegInf) ? 0.f : fast_exp2(x[k] - m_new);
        psum += p;
        __bf16 h = (__bf16)p;
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
      const int qi = lane & 15;
      const char* rlo = vt + (4 * gq + (qi >> 2)) * C::kRowBytes + (qi & 3) * 8;
      const char* rhi = rlo + 16 * C::kRowBytes;
#pragma unroll
      for (int mt = 0; mt < C::kMt; ++mt) {
        bf16x8 vop = tr_pair(rlo + mt * 32, rhi + mt * 32);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, acc[mt], 0, 0, 0);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, acc[mt], 0, 0, 0);
      }
    }

    // finalise: l over the four lanes of head n
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst_o;
    float* dst_l;
    if (whole) {
      dst_o = a.part_o + ((int64_t)bsi * a.Hq + kvh * G) * D;
      dst_l = a.part_lse + (int64_t)bsi * a.Hq + kvh * G;
    } else {
      int32_t slot = piece_slot(w, first);
      dst_o = a.piece_o + (int64_t)slot * G * D;
      dst_l = a.piece_lse + (int64_t)slot * G;
    }
    if (n < G) {
#pragma unroll
      for (int mt = 0; mt < C::kMt; ++mt)
        *(f32x4*)(dst_o + (int64_t)n * D + 16 * mt + 4 * gq) = acc[mt] * inv;
      if (gq == 0) dst_l[n] = l > 0.f ? (m_run + fast_log2(l)) * kLn2 : kNegInf;
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
