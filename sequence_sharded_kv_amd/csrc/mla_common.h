// Helpers shared by the MLA partial-attention kernels (latent rows of 576 bf16: 512 latent
// dims, which are also the value, then 64 rope dims).
#pragma once

#include "device_common.h"

namespace dcp {

constexpr int kMlaDqk = 576;
constexpr int kMlaDv = 512;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// Token permutation inside a 16-row subtile of an LDS tile: MFMA row m holds token pi(m),
// pi(8c + 4h + e) = 8c + h + 2e. The K reads of 8 consecutive MFMA rows then touch 8
// different 16-byte bank groups, and each transposed V read (4 MFMA rows e = 0..3) reads rows
// 2 apart.
__device__ __forceinline__ int tok_of_row(int m) {
  return (m & 8) | ((m >> 2) & 1) | ((m & 3) << 1);
}

// LDS tile of the 64- and 128-row MLA kernels: 32 latent rows in 36 KB, no padding. Region A
// holds dims 0..511, row r at 1024 r; region B dims 512..575, row r at 32768 + 128 r. The
// 16-byte chunk c of row r sits at c ^ mla_swz_a(r) in region A and at c ^ swz_b(r) in region
// B (the HBM -> LDS copies permute the chunks: lane i of a row copy fetches chunk
// i ^ swz(r)). MFMA row m of a 16-row subtile holds token tok_of_row(m). With 512 bytes of
// LDS served per clock (the bank-conflict counter agrees with that model and not with 256),
// the score reads of a half-wave (16 rows x 2 chunks) then cover 32 distinct 16-byte bank
// groups. For the value product the transposed reads of lane group gq (16 lanes) take dims
// 16 mt + 128 (gq & 1) + 4 e of rows 8 (gq >> 1) + 2 i + s2, which leaves them 2-way
// conflicted in half of the wave (SQ_LDS_BANK_CONFLICT about half of that with
// c ^ (r & 15)); a fully conflict-free mapping (32 consecutive dims per block, groups 16 dims
// apart) measured 2.5% slower in the same runs.
__device__ __forceinline__ int mla_swz_a(int r) { return (2 * (r & 15)) ^ (32 * ((r >> 3) & 1)); }
__device__ __forceinline__ int swz_b(int r) { return r & 7; }

// Two transposed 8-byte LDS reads (ds_read_b64_tr_b16) joined into one 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8 mla_tr_pair(const char* lo, const char* hi) {
  i16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)lo);
  i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)hi);
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  i16x8 z = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return __builtin_bit_cast(bf16x8, z);
}

// max / sum over the four lanes n, n+16, n+32, n+48 that hold one head, with the VALU lane
// swaps of gfx950 (cross-lane LDS operations would queue behind the tile reads)
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// One 16-byte-per-lane HBM -> LDS copy from a wave-uniform 64-bit base in scalar registers
// plus a 32-bit per-lane byte offset (the SADDR form of global_load_lds_dwordx4): one VALU
// operation per copy for the offset instead of a 64-bit address per lane. Lane i's 16 bytes
// land at lds_addr + 16 i. The non-temporal policy, the M0 handling and the explicit waits are
// as for dma16.
__device__ __forceinline__ void dma16s(uint64_t sbase, uint32_t voff, uint32_t lds_addr) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);  // wave-uniform by contract
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2 nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(m0v)
      : "memory");
}

// Compute units of `device` (256 on MI355X when the query fails).
inline int mla_cus(int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

}  // namespace dcp
