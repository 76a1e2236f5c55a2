// Device helpers shared by the kernels: stream-K work ranges, piece slots, numerics.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcp_internal.h"

namespace dcp {

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) int32_t i32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// ------------------------------------------------------------------ work split

// First page of worker w's range: floor(w * T / P).
__device__ __forceinline__ int64_t worker_begin(int64_t T, int32_t P, int32_t w) {
  return (int64_t)w * T / P;
}

// The worker whose range contains page g: the largest w with floor(w*T/P) <= g, i.e.
// floor(((g+1)*P - 1) / T), clamped to P-1.
__device__ __forceinline__ int32_t worker_of(int64_t T, int32_t P, int64_t g) {
  int64_t w = ((g + 1) * (int64_t)P - 1) / T;
  return (int32_t)(w < P - 1 ? w : P - 1);
}

// Largest u in [0, U) with pre[u] <= g (pre non-decreasing, pre[0] = 0 <= g < pre[U]).
__device__ __forceinline__ int32_t find_unit(const int32_t* __restrict__ pre, int32_t U, int64_t g) {
  int32_t lo = 0, hi = U - 1;
  while (lo < hi) {
    int32_t mid = (lo + hi + 1) >> 1;
    if ((int64_t)pre[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Slot of the piece that worker w writes for a unit it covers only in part: its first
// segment goes to 2w, its last segment (when that is not also its first) to 2w+1.
__device__ __forceinline__ int32_t piece_slot(int32_t w, bool first_segment) {
  return 2 * w + (first_segment ? 0 : 1);
}

// ------------------------------------------------------------------ LDS copies

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, l);
  uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

// Queue one 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane i's 16 bytes
// land at LDS byte address lds_addr + 16 i. Written as inline asm so that the compiler does
// not treat every later LDS read as possibly overwritten by it (it would otherwise wait for
// the next tile's copies before the first transposed read of the current tile); completion
// is awaited explicitly with vmcnt(0) before the barrier that publishes a tile. M0 is saved
// and restored. The copy carries the non-temporal cache policy: every KV byte is read once
// per step. In a copy-only probe at 2-8 waves per CU, HBM then delivers 6.7-6.9 TB/s against
// 5.2-5.8 TB/s with the default policy. The MLA kernels gain about 1%, because the depth of
// copies in flight bounds them rather than the stream rate.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // wave-uniform by contract
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(m0v)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}

// ------------------------------------------------------------------ numerics

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// LSE merge of (lse_a, o_a) and (lse_b, o_b) is done by callers with these weights:
// given M = max lse, w_k = exp(lse_k - M); all-empty (M = -inf) gives w = 0.
__device__ __forceinline__ float safe_exp_diff(float a, float m) {
  return (m == kNegInf) ? 0.f : __expf(a - m);
}

}  // namespace dcp
