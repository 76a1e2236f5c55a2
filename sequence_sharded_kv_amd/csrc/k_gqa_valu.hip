// GQA partial attention on the vector ALUs, for fp32 caches and shapes the MFMA kernel does
// not take (group size <= 16, head_dim a multiple of 64 up to 256).
//
// Each wave is one stream-K worker. Per 64-token tile, lane t scores token t against the G
// query heads of its KV head (q broadcast from LDS), the per-head tile max and the running
// sums use wave shuffles, and the P.V product switches to lanes-over-dims: the tile's
// probabilities go through LDS and every lane accumulates its dims of O over the 64 tokens,
// with each token's V row address taken from the lane that looked up its page.
#include "device_common.h"

namespace dcp {

constexpr int kValuWaves = 2;  // keeps dynamic LDS <= 40 KB
constexpr int kValuMaxG = 16;
constexpr int kValuVBatch = 4;  // V rows whose loads are in flight together

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(const float* p, int64_t i) { return p[i]; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
  }
};

// Eight consecutive elements from p + i (i a multiple of 8, p 16-byte aligned) with 128-bit
// loads.
__device__ __forceinline__ void load8(const float* p, int64_t i, float* out) {
  const f32x4 a0 = *(const f32x4*)(p + i), a1 = *(const f32x4*)(p + i + 4);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j] = a0[j];
    out[4 + j] = a1[j];
  }
}
__device__ __forceinline__ void load8(const uint16_t* p, int64_t i, float* out) {
  const u32x4 w = *(const u32x4*)(p + i);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <typename T, int NDV>  // NDV = head_dim / 64
__global__ void __launch_bounds__(64 * kValuWaves)
gqa_valu_kernel(AttnArgs a) {
  extern __shared__ float valu_lds[];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int D = NDV * 64;
  float* qs = valu_lds + wv * (kValuMaxG * D + kValuMaxG * 64);  // [G][D]
  float* ps = qs + kValuMaxG * D;                                 // [G][64]
  const int32_t w = blockIdx.x * kValuWaves + wv;
  if (w >= a.P) return;
  const T* __restrict__ Q = (const T*)a.q;
  const T* __restrict__ K = (const T*)a.k;
  const T* __restrict__ V = (const T*)a.v;
  const int64_t T_pages = a.pre[a.U];
  const int64_t g0 = worker_begin(T_pages, a.P, w), g1 = worker_begin(T_pages, a.P, w + 1);
  if (g0 >= g1) return;
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
    const int32_t Ru = a.Ru;
    const int64_t ta = a.ubounds[2 * bsi], te = a.ubounds[2 * bsi + 1];
    const int64_t pa = ta / a.bs;
    int64_t t0 = (pa + (g - up0)) * a.bs, t1 = (pa + (sg1 - up0)) * a.bs;
    if (t0 < ta) t0 = ta;
    if (t1 > te) t1 = te;
    const bool whole = (g == up0) && (sg1 == up1);
    const bool first = (g == g0);
    // the unit's query rows -> LDS (padding rows read as zeros)
    for (int i = lane; i < Ru * D; i += 64) {
      int h = i / D, d = i % D;
      int32_t jh = 0;
      const int32_t rho = unit_row(a, kvh, rg, h, &jh);
      qs[i] = rho >= 0 ? Elem<T>::get(Q, call_row(a, b, rho) * a.Dqk + d) : 0.f;
    }
    // last context position each row may see (several query tokens)
    int32_t lim[kValuMaxG];
#pragma unroll
    for (int h = 0; h < kValuMaxG; ++h) {
      int32_t jh = 0;
      const bool ok = unit_row(a, kvh, rg, h, &jh) >= 0;
      lim[h] = (a.Rs == a.Hq || !ok) ? INT32_MAX : a.qend[b] + a.j0 + jh;
    }
    __builtin_amdgcn_wave_barrier();
    float m[kValuMaxG], lsum[kValuMaxG], acc[kValuMaxG][NDV];
#pragma unroll
    for (int h = 0; h < kValuMaxG; ++h) {
      m[h] = kNegInf;
      lsum[h] = 0.f;
#pragma unroll
      for (int j = 0; j < NDV; ++j) acc[h][j] = 0.f;
    }
    const int32_t* brow = a.block_table + (int64_t)b * a.max_blocks;
    for (int64_t tile = t0; tile < t1; tile += 64) {
      const int64_t t = tile + lane;
      bool valid = t < t1;
      int64_t row = 0;
      if (valid) {
        int32_t blk = brow[t / a.bs];
        if (blk < 0 || blk >= a.num_blocks) { valid = false; bad = 1; }
        else row = (((int64_t)blk * a.Hkv + kvh) * a.bs + t % a.bs) * D;
      }
      float s[kValuMaxG];
#pragma unroll
      for (int h = 0; h < kValuMaxG; ++h) s[h] = 0.f;
      if (valid) {
        for (int d = 0; d < D; d += 8) {
          float kv[8];
          load8(K, row + d, kv);
#pragma unroll
          for (int h = 0; h < kValuMaxG; ++h) {
            if (h < Ru) {
#pragma unroll
              for (int j = 0; j < 8; ++j) s[h] = fmaf(qs[h * D + d + j], kv[j], s[h]);
            }
          }
        }
      }
      const int nvalid = (int)((t1 - tile) < 64 ? (t1 - tile) : 64);
#pragma unroll
      for (int h = 0; h < kValuMaxG; ++h) {
        if (h < Ru) {
          float x = (valid && t <= lim[h]) ? s[h] * a.scale_log2 : kNegInf;
          float mn = fmaxf(m[h], wave_max(x));
          float alpha = (mn == kNegInf) ? 1.f : fast_exp2(m[h] - mn);
          float p = (x == kNegInf) ? 0.f : fast_exp2(x - mn);
          lsum[h] = lsum[h] * alpha + p;
          ps[h * 64 + lane] = p;
#pragma unroll
          for (int j = 0; j < NDV; ++j) acc[h][j] *= alpha;
          m[h] = mn;
        }
      }
      __builtin_amdgcn_wave_barrier();
      // V rows of the tile's tokens, kValuVBatch at a time: token tt's row (K and V share the
      // cache layout) comes from lane tt, so no table load sits in this loop, and the batch's
      // loads are in flight together; tokens without a valid row are skipped (their weight is
      // zero, and their row may hold anything)
      const uint64_t vmask = __ballot(valid);
      for (int tt0 = 0; tt0 < nvalid; tt0 += kValuVBatch) {
        float vv[kValuVBatch][NDV];
#pragma unroll
        for (int k = 0; k < kValuVBatch; ++k) {
          const int tt = tt0 + k;  // wave-uniform
          const bool use = tt < nvalid && ((vmask >> tt) & 1u);
          const int64_t vrow = (int64_t)readlane_u64((uint64_t)row, tt < 64 ? tt : 0);
#pragma unroll
          for (int j = 0; j < NDV; ++j)
            vv[k][j] = use ? Elem<T>::get(V, vrow + lane + 64 * j) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < kValuVBatch; ++k) {
          const int tt = tt0 + k;
          if (tt >= nvalid) break;
#pragma unroll
          for (int h = 0; h < kValuMaxG; ++h) {
            if (h < Ru) {
              const float p = ps[h * 64 + tt];
#pragma unroll
              for (int j = 0; j < NDV; ++j) acc[h][j] = fmaf(p, vv[k][j], acc[h][j]);
            }
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    // finalise and write this segment's partial
    const int32_t slot = piece_slot(w, first);
#pragma unroll
    for (int h = 0; h < kValuMaxG; ++h) {
      int32_t jh = 0;
      const int32_t rho = unit_row(a, kvh, rg, h, &jh);
      if (rho >= 0) {
        float* dst_o = whole ? a.part_o + part_row(a, bsi, rho) * a.Dv
                             : a.piece_o + ((int64_t)slot * Ru + h) * a.Dv;
        float* dst_l = whole ? a.part_lse + part_row(a, bsi, rho)
                             : a.piece_lse + (int64_t)slot * Ru + h;
        float l = wave_sum(lsum[h]);
        float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int j = 0; j < NDV; ++j) dst_o[lane + 64 * j] = acc[h][j] * inv;
        if (lane == 0) *dst_l = l > 0.f ? (m[h] + fast_log2(l)) * kLn2 : kNegInf;
      }
    }
    __builtin_amdgcn_wave_barrier();
    g = sg1;
  }
  if (bad) atomicOr(a.flags, kFlagBadBlock);
}

int32_t gqa_valu_workers(int device, int32_t max_workers) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  int32_t p = cus * kValuWaves * 2;
  return p < max_workers ? p : max_workers;
}

template <typename T, int NDV>
static hipError_t launch_valu_t(const AttnArgs& a, hipStream_t stream) {
  size_t lds = (size_t)kValuWaves * (kValuMaxG * NDV * 64 + kValuMaxG * 64) * sizeof(float);
  int32_t grid = (a.P + kValuWaves - 1) / kValuWaves;
  hipLaunchKernelGGL((gqa_valu_kernel<T, NDV>), dim3(grid), dim3(64 * kValuWaves), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_gqa_valu(const AttnArgs& a, int32_t dtype, hipStream_t stream) {
  const int ndv = a.Dqk / 64;
  if (dtype == DCP_F32) {
    switch (ndv) {
      case 1: return launch_valu_t<float, 1>(a, stream);
      case 2: return launch_valu_t<float, 2>(a, stream);
      case 3: return launch_valu_t<float, 3>(a, stream);
      case 4: return launch_valu_t<float, 4>(a, stream);
    }
  } else {
    switch (ndv) {
      case 1: return launch_valu_t<uint16_t, 1>(a, stream);
      case 2: return launch_valu_t<uint16_t, 2>(a, stream);
      case 3: return launch_valu_t<uint16_t, 3>(a, stream);
      case 4: return launch_valu_t<uint16_t, 4>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace dcp
