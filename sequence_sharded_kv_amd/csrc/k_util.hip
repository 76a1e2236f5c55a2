// Small kernels around the partial-attention kernels: device shard plan, work schedule,
// per-unit finishing (merging the pieces of units cut by worker boundaries), the LSE merge
// across shards, and the debug page gather.
#include "device_common.h"

namespace dcp {

// ---------------------------------------------------------------- device shard plan

// Canonical plan (page-aligned ceil split, see dcp_plan_shards in dcp.h): one thread per
// (request, shard).
__global__ void plan_device_kernel(const int32_t* __restrict__ seq_lens, int32_t B, int32_t S,
                                   int32_t bs, int32_t* __restrict__ bounds) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)B * S) return;
  int32_t b = (int32_t)(i / S), s = (int32_t)(i % S);
  int64_t L = seq_lens[b];
  if (L < 0) L = 0;
  int64_t pages = (L + bs - 1) / bs;
  int64_t per = (pages + S - 1) / S;
  int64_t a = (int64_t)s * per * bs, e = (int64_t)(s + 1) * per * bs;
  bounds[2 * i] = (int32_t)(a < L ? a : L);
  bounds[2 * i + 1] = (int32_t)(e < L ? e : L);
}

hipError_t launch_plan_device(const int32_t* seq_lens, int32_t B, int32_t S, int32_t bs,
                              int32_t* bounds, hipStream_t stream) {
  int64_t n = (int64_t)B * S;
  int32_t grid = (int32_t)((n + 255) / 256);
  hipLaunchKernelGGL(plan_device_kernel, dim3(grid), dim3(256), 0, stream, seq_lens, B, S, bs,
                     bounds);
  return hipGetLastError();
}

// ---------------------------------------------------------------- schedule

// One workgroup: sanitise the bounds of every (request, shard), count each unit's pages and
// write the exclusive prefix sum pre[0..U] (units ordered (b, s, h) with h < units_per_bs).
// A second pass lists the units the finishing pass must write (cut by a worker boundary, or
// without pages) in `fin`, with their count in flags[1], and records who wrote each unit in
// `usrc` (for the combining pass). Also clears the
// flag word (the first call of a step owns it) and the P recomputation marks.
constexpr int kSchedThreads = 1024;
constexpr int kSchedPer = 4;  // consecutive units per thread in one pass of the scan

__global__ void __launch_bounds__(kSchedThreads)
schedule_kernel(const int32_t* __restrict__ bounds, int32_t B, int32_t S, int32_t units_per_bs,
                int32_t P, int32_t* __restrict__ fin, int32_t bs, int32_t max_blocks,
                int32_t* __restrict__ ubounds, int32_t* __restrict__ pre,
                int32_t* __restrict__ flags, int32_t Tq, int32_t* __restrict__ qend,
                int32_t* __restrict__ redo, int32_t* __restrict__ usrc, int32_t keep_flags) {
  __shared__ int32_t warp_sums[kSchedThreads / 64];
  __shared__ int32_t carry;
  __shared__ int32_t flag_acc;
  __shared__ int32_t fin_count;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  if (tid == 0) { carry = 0; flag_acc = 0; fin_count = 0; }
  for (int i = tid; i < kWsZeroWords; i += kSchedThreads) flags[kWsZeroOffset / 4 + i] = 0;
  for (int i = tid; i < P; i += kSchedThreads) redo[i] = 0;
  __syncthreads();
  const int64_t cap = (int64_t)max_blocks * bs;
  const int64_t nbs = (int64_t)B * S;
  const int64_t U = nbs * units_per_bs;
  // consecutive units per thread: as few as cover the units in one pass (up to kSchedPer)
  const int32_t per = U <= kSchedThreads ? 1 : U <= 2 * kSchedThreads ? 2 : kSchedPer;
  const int64_t pass = (int64_t)kSchedThreads * per;
  int32_t my_flag = 0;
  // page offsets and counts of this thread's units in the last pass (all of them when one
  // pass covers every unit)
  int32_t p0s[kSchedPer], cnts[kSchedPer];
  for (int64_t base = 0; base < U; base += pass) {
    // U * max_blocks fits in 32 bits (checked by the host plan), so unit indices do too
    const int64_t u0 = base + (int64_t)tid * per;
    int32_t tot = 0;
#pragma unroll
    for (int k = 0; k < kSchedPer; ++k) {
      const int64_t u = u0 + k;
      cnts[k] = 0;
      if (k < per && u < U) {
        const int64_t bsi = (int64_t)((uint32_t)u / (uint32_t)units_per_bs);
        int64_t a = bounds[2 * bsi], e = bounds[2 * bsi + 1];
        const int64_t a0 = a, e0 = e;
        if (a < 0) a = 0;
        if (e > cap) e = cap;
        if (a > cap) a = cap;
        if (e < a) e = a;
        if (a != a0 || e != e0) my_flag |= kFlagBoundClamped;
        if ((uint32_t)u - (uint32_t)bsi * (uint32_t)units_per_bs == 0) {
          ubounds[2 * bsi] = (int32_t)a;
          ubounds[2 * bsi + 1] = (int32_t)e;
        }
        // 0 <= a <= e <= cap <= INT32_MAX: 32-bit page arithmetic
        cnts[k] = (e > a) ? (int32_t)(((uint32_t)e + (uint32_t)bs - 1u) / (uint32_t)bs -
                                      (uint32_t)a / (uint32_t)bs)
                          : 0;
      }
      tot += cnts[k];
    }
    // exclusive scan of the threads' totals: within the wave, then over the waves
    int32_t x = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) warp_sums[wv] = x;
    __syncthreads();
    if (wv == 0) {
      int32_t ws = (lane < kSchedThreads / 64) ? warp_sums[lane] : 0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(ws, off, 64);
        if (lane >= off) ws += y;
      }
      if (lane < kSchedThreads / 64) warp_sums[lane] = ws;  // inclusive over waves
    }
    __syncthreads();
    int32_t run = carry + (wv > 0 ? warp_sums[wv - 1] : 0) + x - tot;
#pragma unroll
    for (int k = 0; k < kSchedPer; ++k) {
      p0s[k] = run;
      if (k < per && u0 + k < U) pre[u0 + k] = run;
      run += cnts[k];
    }
    __syncthreads();  // every thread has read carry
    if (tid == kSchedThreads - 1) carry = run;
    __syncthreads();
  }
  if (my_flag) atomicOr(&flag_acc, my_flag);
  const int64_t T = carry;
  if (tid == 0) pre[U] = (int32_t)T;
  __syncthreads();  // ubounds[] is complete and visible to the workgroup
  // position of each request's first query token: the end of its ranges minus Tq
  for (int64_t b = tid; b < B; b += kSchedThreads) {
    int32_t end = 0;
    for (int32_t sh = 0; sh < S; ++sh) end = max(end, ubounds[2 * (b * S + sh) + 1]);
    qend[b] = end - Tq;
  }
  // worker_of in 32-bit unsigned arithmetic when (T + 1) * P fits (the same quotients; the
  // 64-bit divisions cost more than the rest of this pass)
  const bool narrow = (T + 1) * (int64_t)P < ((int64_t)1 << 32);
  auto owner = [&](int64_t g) -> int32_t {
    if (narrow) {
      const uint32_t w = ((uint32_t)(g + 1) * (uint32_t)P - 1u) / (uint32_t)T;
      return (int32_t)(w < (uint32_t)(P - 1) ? w : (uint32_t)(P - 1));
    }
    return worker_of(T, P, g);
  };
  auto begin_of = [&](int32_t w) -> int64_t {
    if (narrow) return (int64_t)((uint32_t)w * (uint32_t)T / (uint32_t)P);
    return worker_begin(T, P, w);
  };
  // who writes each unit; units cut by worker boundaries or without pages go to `fin`
  auto place = [&](int64_t u, int64_t p0, int64_t p1) {
    int32_t w0 = -1, w1 = -1, slot0 = -1;
    if (p1 > p0) {
      w0 = owner(p0);
      w1 = owner(p1 - 1);
      // the unit is w0's first segment unless w0's range began before it
      slot0 = piece_slot(w0, !(begin_of(w0) < p0));
    }
    *(i32x4*)(usrc + 4 * u) = i32x4{w0, w1, slot0, (int32_t)p0};
    if (p1 > p0 && w0 == w1) return;  // written whole by its worker
    const int32_t k = atomicAdd(&fin_count, 1);
    *(i32x4*)(fin + 4 * (int64_t)k) = i32x4{(int32_t)u, w0, w1, 0};
  };
  if (U <= pass) {
    // one pass: the offsets are still in registers
#pragma unroll
    for (int k = 0; k < kSchedPer; ++k) {
      const int64_t u = (int64_t)tid * per + k;
      if (k < per && u < U) place(u, p0s[k], (int64_t)p0s[k] + cnts[k]);
    }
  } else {
    __syncthreads();  // pre[] is complete and visible to the workgroup
    for (int64_t u = tid; u < U; u += kSchedThreads) place(u, pre[u], pre[u + 1]);
  }
  __syncthreads();
  if (tid == 0) {
    // a later pass of the same call keeps what the earlier passes flagged
    flags[0] = keep_flags ? (flags[0] | flag_acc) : flag_acc;
    flags[1] = fin_count;
  }
}

hipError_t launch_schedule(const int32_t* bounds, int32_t B, int32_t S, int32_t units_per_bs,
                           int32_t P, int32_t* fin, int32_t bs, int32_t max_blocks,
                           int32_t* ubounds, int32_t* pre, int32_t* flags, int32_t Tq,
                           int32_t* qend, int32_t* redo, int32_t* usrc, int32_t keep_flags,
                           hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, bounds, B, S,
                     units_per_bs, P, fin, bs, max_blocks, ubounds, pre, flags, Tq, qend, redo,
                     usrc, keep_flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------- finish units

// Writes the partial of every unit in the schedule's `fin` list. A unit with no pages gets
// O = 0, LSE = -inf. A unit cut by worker boundaries left one piece per covering worker
// (none from a worker whose range is empty); the pieces are merged by the LSE formula.
// Grid (x, c): workgroup x takes list entries x, x + gridDim.x, ...; chunk c is 1024
// consecutive floats of the unit's Ru x Dv rows (one float4 per thread), each written to its
// query row of the partials.
constexpr int kFinishThreads = 256;
constexpr int kFinishMaxPieces = 4096;  // >= the most workers any launch uses
constexpr int kFinishUnroll = 4;        // pieces whose loads are issued together

__global__ void __launch_bounds__(kFinishThreads) __attribute__((amdgpu_waves_per_eu(8)))
finish_units_kernel(AttnArgs a) {
  __shared__ int32_t slots[kFinishMaxPieces];  // -1 for workers that own no pages
  const int32_t count = a.flags[1];
  const int64_t T = a.pre[a.U];
  const int32_t per_bs = a.U / (a.B * a.S);
  const int32_t Hu = a.Ru;
  const int32_t n4 = Hu * a.Dv / 4;
  const int32_t i4 = blockIdx.y * kFinishThreads + threadIdx.x;
  const int32_t h = 4 * i4 / a.Dv;          // local row of the unit
  const int32_t c4 = i4 - h * (a.Dv / 4);   // float4 within the row
  for (int32_t e = blockIdx.x; e < count; e += gridDim.x) {
    const i32x4 ent = *(const i32x4*)(a.fin + 4 * (int64_t)e);
    const int32_t u = ent[0], w0 = ent[1], w1 = ent[2];
    const int32_t bsi = u / per_bs, hsub = u % per_bs;
    int32_t jtok = 0;
    const int32_t rho = (i4 < n4) ? unit_row(a, hsub / a.NRg, hsub % a.NRg, h, &jtok) : -1;
    float* out_o = a.part_o + part_row(a, bsi, rho < 0 ? 0 : rho) * a.Dv;
    float* out_l = a.part_lse + part_row(a, bsi, rho < 0 ? 0 : rho);
    if (w0 < 0) {
      if (rho >= 0) {
        ((f32x4*)out_o)[c4] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (c4 == 0) *out_l = kNegInf;
      }
      continue;
    }
    const int64_t p0 = a.pre[u];
    const int32_t ns = w1 - w0 + 1;
    __syncthreads();  // slots of the previous entry are no longer read
    for (int32_t k = threadIdx.x; k < ns; k += kFinishThreads) {
      const int32_t w = w0 + k;
      const int64_t wb = worker_begin(T, a.P, w);
      slots[k] = (worker_begin(T, a.P, w + 1) == wb) ? -1 : piece_slot(w, !(w == w0 && wb < p0));
    }
    __syncthreads();
    if (rho < 0) continue;
    // One pass over the pieces, kFinishUnroll at a time so that their loads are in flight
    // together: the running max m moves to the batch's max and the sums so far are rescaled
    // by exp(m_old - m_new) (the same re-weighting as the LSE merge).
    float m = kNegInf, den = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int32_t k0 = 0; k0 < ns; k0 += kFinishUnroll) {
      float lb[kFinishUnroll];
      f32x4 ob[kFinishUnroll];
#pragma unroll
      for (int j = 0; j < kFinishUnroll; ++j) {
        const int32_t sl = (k0 + j < ns) ? slots[k0 + j] : -1;
        lb[j] = kNegInf;
        ob[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sl >= 0) {
          lb[j] = a.piece_lse[(int64_t)sl * Hu + h];
          ob[j] = ((const f32x4*)(a.piece_o + (int64_t)sl * Hu * a.Dv))[i4];
        }
      }
      float mb = m;
#pragma unroll
      for (int j = 0; j < kFinishUnroll; ++j) mb = fmaxf(mb, lb[j]);
      const float sc = safe_exp_diff(m, mb);  // 0 while both are -inf (nothing summed yet)
      den *= sc;
      acc *= sc;
#pragma unroll
      for (int j = 0; j < kFinishUnroll; ++j) {
        const float wt = safe_exp_diff(lb[j], mb);
        den += wt;
        acc += wt * ob[j];
      }
      m = mb;
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
    ((f32x4*)out_o)[c4] = acc * inv;
    if (c4 == 0) *out_l = den > 0.f ? m + logf(den) : kNegInf;
  }
}

hipError_t launch_finish_units(const AttnArgs& a, hipStream_t stream) {
  if (a.U == 0) return hipSuccess;
  if (a.P > kFinishMaxPieces) return hipErrorInvalidValue;
  const int32_t n4 = a.Ru * a.Dv / 4;
  const int32_t chunks = (n4 + kFinishThreads - 1) / kFinishThreads;
  int32_t x = (4096 + chunks - 1) / chunks;
  if (x > a.U) x = a.U;
  hipLaunchKernelGGL(finish_units_kernel, dim3(x, chunks), dim3(kFinishThreads), 0, stream, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- LSE merge

// out[b, h, :] = sum_s exp(LSE_s - LSE) O_s with LSE = M + ln sum_s exp(LSE_s - M).
// One thread per 4 output values; a workgroup covers 256 x 4 values of one or more heads.
constexpr int32_t kMergeUnroll = 16;  // shard counts up to this keep every load in flight
__global__ void __launch_bounds__(256)
merge_kernel(int32_t B, int32_t S, int32_t H, int32_t Dv, const float* __restrict__ part_o,
             const float* __restrict__ part_lse, float* __restrict__ out,
             float* __restrict__ out_lse) {
  const int64_t q4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // float4 index
  const int32_t dv4 = Dv >> 2;
  if (q4 >= (int64_t)B * H * dv4) return;
  const int64_t bh = q4 / dv4;
  const int32_t c = (int32_t)(q4 % dv4);
  const int64_t b = bh / H, h = bh % H;
  const float* lse = part_lse + b * S * H + h;
  const float* po = part_o + (b * S * H + h) * Dv + 4 * c;
  const int64_t so = (int64_t)H * Dv;  // stride between shards
  float m = kNegInf;
  float den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // A shard with zero weight (LSE = -inf) contributes nothing whatever its O holds.
  auto add = [&](float l, const f32x4& o) {
    const float w = safe_exp_diff(l, m);
    den += w;
    if (w != 0.f) acc += w * o;
  };
  if (S <= kMergeUnroll) {
    // all 2 S loads queued before the first use
    float l[kMergeUnroll];
    f32x4 o[kMergeUnroll];
#pragma unroll
    for (int32_t s = 0; s < kMergeUnroll; ++s)
      if (s < S) {
        l[s] = lse[(int64_t)s * H];
        o[s] = *(const f32x4*)(po + s * so);
      }
#pragma unroll
    for (int32_t s = 0; s < kMergeUnroll; ++s)
      if (s < S) m = fmaxf(m, l[s]);
#pragma unroll
    for (int32_t s = 0; s < kMergeUnroll; ++s)
      if (s < S) add(l[s], o[s]);
  } else {
    for (int32_t s = 0; s < S; ++s) m = fmaxf(m, lse[(int64_t)s * H]);
    for (int32_t s = 0; s < S; ++s) add(lse[(int64_t)s * H], *(const f32x4*)(po + s * so));
  }
  float inv = den > 0.f ? 1.f / den : 0.f;
  *(f32x4*)(out + bh * Dv + 4 * c) = acc * inv;
  if (out_lse && c == 0) out_lse[bh] = den > 0.f ? m + logf(den) : kNegInf;
}

hipError_t launch_merge(int32_t B, int32_t S, int32_t H, int32_t Dv, const float* part_o,
                        const float* part_lse, float* out, float* out_lse, hipStream_t stream) {
  int64_t n = (int64_t)B * H * (Dv / 4);
  int32_t grid = (int32_t)((n + 255) / 256);
  hipLaunchKernelGGL(merge_kernel, dim3(grid), dim3(256), 0, stream, B, S, H, Dv, part_o,
                     part_lse, out, out_lse);
  return hipGetLastError();
}

// ---------------------------------------------------------------- combine (fused calls)

// out[b, rho, :] and out_lse[b, rho] of the fused calls straight from the attention kernel's
// outputs, without the finishing pass: for each shard, the unit holding query row rho
// contributes its partial row when one worker wrote it whole, the rows of its pieces when
// worker boundaries cut it (one per covering worker whose range is not empty), and nothing
// when it has no pages. All of them enter one LSE merge, which is associative: the result is
// that of merging the pieces into each shard's partial and the partials into the output, up
// to rounding order. kSplit consecutive threads share one output float4: thread t takes the
// shards s = t (mod kSplit) and, of each cut unit, the pieces j = t (mod kSplit), and the
// group's partial merges are combined across its lanes at the end (the same formula). A
// thread issues its sources' loads kB at a time. kSplit > 1 serves launches with few output
// values and many pieces per value, which one thread per value would walk through one memory
// latency per batch.
template <int kSplit, int kB>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
combine_kernel(AttnArgs a, float* __restrict__ out, float* __restrict__ out_lse) {
  const int32_t dv4 = a.Dv >> 2;
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int32_t t = (int32_t)(q % kSplit);
  const int64_t q4 = q / kSplit;
  // the groups' lanes stay together to the end (kSplit divides the wave): no early exit
  const bool live = q4 < (int64_t)a.B * a.R * dv4;
  const int64_t br = live ? q4 / dv4 : 0;  // b * R + rho
  const int32_t c4 = live ? (int32_t)(q4 - br * dv4) : 0;
  const int32_t b = (int32_t)(br / a.R), rho = (int32_t)(br - (int64_t)b * a.R);
  // the unit column and local row of query row rho = j Hq + kvh G + g (inverse of unit_row)
  const int32_t jq = rho / a.Hq, hq = rho - jq * a.Hq;
  const int32_t kvh = hq / a.G;
  const int32_t rr = jq * a.G + (hq - kvh * a.G);
  const int32_t rg = rr / a.Ru, h = rr - rg * a.Ru;
  const int32_t per_bs = a.U / (a.B * a.S);
  const int64_t col = (int64_t)kvh * a.NRg + rg;
  const i32x4* usrc = (const i32x4*)a.usrc;
  // with at least as many pages as workers no worker's range is empty; with fewer, each
  // worker's range holds at most one page, and the pieces of a unit are its pages' owners
  const int64_t T = a.pre[a.U];
  const bool all_ranges = T >= a.P;
  float m = kNegInf, den = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  // one batch of sources: the running max moves to the batch's max and the sums so far are
  // rescaled by exp(m_old - m_new); a zero weight takes no part, whatever its O holds
  auto merge = [&](const float* l, const f32x4* o) {
    float mb = m;
#pragma unroll
    for (int c = 0; c < kB; ++c) mb = fmaxf(mb, l[c]);
    const float sc = safe_exp_diff(m, mb);
    den *= sc;
    acc *= sc;
#pragma unroll
    for (int c = 0; c < kB; ++c) {
      const float wt = safe_exp_diff(l[c], mb);
      den += wt;
      if (wt != 0.f) acc += wt * o[c];
    }
    m = mb;
  };
  for (int32_t s0 = 0; live && s0 < a.S; s0 += kB) {
    i32x4 src[kB];
#pragma unroll
    for (int c = 0; c < kB; ++c)
      src[c] = s0 + c < a.S ? usrc[((int64_t)b * a.S + s0 + c) * per_bs + col]
                            : i32x4{-1, -1, -1, 0};
    // units written whole: their partial rows. The rows are loaded alongside the table (the
    // workspace rows of the other units hold whatever an earlier call left) and weighted
    // only where the table says one worker wrote the unit.
    float l[kB];
    f32x4 o[kB];
#pragma unroll
    for (int c = 0; c < kB; ++c) {
      l[c] = kNegInf;
      o[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s0 + c < a.S && (s0 + c) % kSplit == t) {
        const int64_t row = part_row(a, (int64_t)b * a.S + s0 + c, rho);
        l[c] = a.part_lse[row];
        o[c] = *(const f32x4*)(a.part_o + row * a.Dv + 4 * c4);
      }
    }
#pragma unroll
    for (int c = 0; c < kB; ++c)
      if (!(src[c][0] >= 0 && src[c][0] == src[c][1])) l[c] = kNegInf;
    merge(l, o);
    // units cut by worker boundaries: their pieces
#pragma unroll
    for (int c = 0; c < kB; ++c) {
      const int32_t w0 = src[c][0], w1 = src[c][1];
      if (w0 < 0 || w0 == w1) continue;
      // pieces j = 0 .. n - 1: the covering workers in order, or the unit's pages' owners
      const int64_t p0 = src[c][3];
      const int32_t n = all_ranges ? w1 - w0 + 1 : (int32_t)((int64_t)w1 * T / a.P + 1 - p0);
      for (int32_t j0 = t; j0 < n; j0 += kB * kSplit) {
#pragma unroll
        for (int k = 0; k < kB; ++k) {
          const int32_t jj = j0 + k * kSplit;
          l[k] = kNegInf;
          o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (jj < n) {
            // the unit is the first segment of every covering worker but w0, whose slot the
            // schedule recorded
            const int32_t w = all_ranges || jj == 0 ? w0 + jj : worker_of(T, a.P, p0 + jj);
            const int64_t sl = jj == 0 ? src[c][2] : piece_slot(w, true);
            l[k] = a.piece_lse[sl * a.Ru + h];
            o[k] = *(const f32x4*)(a.piece_o + (sl * a.Ru + h) * a.Dv + 4 * c4);
          }
        }
        merge(l, o);
      }
    }
  }
  // the group's partial merges, combined across its lanes
#pragma unroll
  for (int off = 1; off < kSplit; off <<= 1) {
    const float m2 = __shfl_xor(m, off, 64);
    const float d2 = __shfl_xor(den, off, 64);
    f32x4 a2;
#pragma unroll
    for (int e = 0; e < 4; ++e) a2[e] = __shfl_xor(acc[e], off, 64);
    const float mb = fmaxf(m, m2);
    const float s1 = safe_exp_diff(m, mb), s2 = safe_exp_diff(m2, mb);
    den = den * s1 + d2 * s2;
    acc = (s1 != 0.f ? acc * s1 : f32x4{0.f, 0.f, 0.f, 0.f}) +
          (s2 != 0.f ? a2 * s2 : f32x4{0.f, 0.f, 0.f, 0.f});
    m = mb;
  }
  if (!live || t != 0) return;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t orow = call_row(a, b, rho);  // the caller's row (a pass may start at j0 > 0)
  *(f32x4*)(out + orow * a.Dv + 4 * c4) = acc * inv;
  if (out_lse && c4 == 0) out_lse[orow] = den > 0.f ? m + logf(den) : kNegInf;
}

hipError_t launch_combine(const AttnArgs& a, float* out, float* out_lse, hipStream_t stream) {
  const int64_t n = (int64_t)a.B * a.R * (a.Dv / 4);
  if (n == 0) return hipSuccess;
  // few output values: eight threads per value, so that the launch has about as many
  // threads as the one-per-value launch of a large batch
  if (n < (int64_t)1 << 19) {
    const int32_t grid = (int32_t)((8 * n + 255) / 256);
    hipLaunchKernelGGL((combine_kernel<8, 2>), dim3(grid), dim3(256), 0, stream, a, out,
                       out_lse);
  } else {
    const int32_t grid = (int32_t)((n + 255) / 256);
    hipLaunchKernelGGL((combine_kernel<1, 8>), dim3(grid), dim3(256), 0, stream, a, out,
                       out_lse);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- debug gather

__global__ void debug_gather_kernel(const uint8_t* __restrict__ cache,
                                    const int32_t* __restrict__ block_table,
                                    const int32_t* __restrict__ bounds, int32_t S, int32_t b,
                                    int32_t s, int32_t kv_head, int32_t Hkv, int32_t bs,
                                    int32_t max_blocks, int32_t num_blocks, int32_t row_bytes,
                                    int32_t gqa, uint8_t* __restrict__ dst, int32_t max_rows) {
  int64_t cap = (int64_t)max_blocks * bs;
  int64_t a = bounds[2 * ((int64_t)b * S + s)], e = bounds[2 * ((int64_t)b * S + s) + 1];
  if (a < 0) a = 0;
  if (e > cap) e = cap;
  if (a > cap) a = cap;
  if (e < a) e = a;
  int64_t n = e - a;
  if (n > max_rows) n = max_rows;
  for (int64_t r = blockIdx.x; r < n; r += gridDim.x) {
    int64_t t = a + r;
    int32_t blk = block_table[(int64_t)b * max_blocks + t / bs];
    int32_t slot = (int32_t)(t % bs);
    uint8_t* d = dst + r * row_bytes;
    if (blk < 0 || blk >= num_blocks) {
      for (int32_t i = threadIdx.x; i < row_bytes; i += blockDim.x) d[i] = 0;
      continue;
    }
    int64_t row = gqa ? (((int64_t)blk * Hkv + kv_head) * bs + slot) : ((int64_t)blk * bs + slot);
    const uint8_t* src = cache + row * row_bytes;
    for (int32_t i = threadIdx.x; i < row_bytes; i += blockDim.x) d[i] = src[i];
  }
}

hipError_t launch_debug_gather(const dcp_attn_shape& sh, const void* cache,
                               const int32_t* block_table, const int32_t* bounds, int32_t b,
                               int32_t s, int32_t kv_head, void* dst, int32_t max_rows,
                               hipStream_t stream) {
  int32_t esize = sh.dtype == DCP_F32 ? 4 : 2;
  int32_t row_bytes = sh.head_dim_qk * esize;
  hipLaunchKernelGGL(debug_gather_kernel, dim3(256), dim3(256), 0, stream,
                     (const uint8_t*)cache, block_table, bounds, sh.num_shards, b, s, kv_head,
                     sh.num_kv_heads, sh.block_size, sh.max_blocks_per_seq, sh.num_blocks,
                     row_bytes, sh.kv_kind == DCP_KV_GQA ? 1 : 0, (uint8_t*)dst, max_rows);
  return hipGetLastError();
}


// ---------------------------------------------------------------- KV append

// One workgroup per request stores the token it decoded this step. A request holding L tokens
// writes position L: slot L % bs of page block_table[b][L / bs]. Its owner is the shard whose
// range in the plan of L + 1 tokens contains L: with p = L / bs that plan has p + 1 pages and
// k = ceil((p + 1) / S) pages per shard, so the owner is p / k. Rows move as 16-byte chunks:
// kc (and vc) chunks per head, Hkv heads (1 for the MLA latent cache, vc = 0). The first
// chunk of each thread is loaded before the length and the table entry are known, so its
// latency overlaps theirs instead of following them.
constexpr int32_t kAppendThreads = 128;

__global__ void __launch_bounds__(kAppendThreads)
append_kv_kernel(const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table,
                 const i32x4* __restrict__ new_k, const i32x4* __restrict__ new_v,
                 i32x4* __restrict__ k_cache, i32x4* __restrict__ v_cache,
                 int32_t* __restrict__ owner, int32_t Hkv, int32_t kc, int32_t vc, int32_t bs,
                 int32_t max_blocks, int32_t num_blocks, int32_t S) {
  const int32_t b = blockIdx.x;
  const int32_t per_head = kc + vc;
  const int32_t total = Hkv * per_head;
  auto src_of = [&](int32_t i) -> i32x4 {
    const int32_t h = i / per_head, j = i - h * per_head;
    const int64_t src = (int64_t)b * Hkv + h;
    return j < kc ? new_k[src * kc + j] : new_v[src * vc + (j - kc)];
  };
  const int32_t i0 = threadIdx.x;
  i32x4 first = {0, 0, 0, 0};
  if (i0 < total) first = src_of(i0);

  const int32_t L = seq_lens[b];
  const int32_t p = L >= 0 ? L / bs : 0;
  int32_t who = -1;
  int32_t blk = 0;
  if (L >= 0 && p < max_blocks) {
    blk = block_table[(int64_t)b * max_blocks + p];
    if (blk < 0 || blk >= num_blocks) {
      who = -2;
    } else {
      const uint32_t per_shard = ((uint32_t)p + (uint32_t)S) / (uint32_t)S;  // < 2^32: p, S < 2^31
      who = (int32_t)((uint32_t)p / per_shard);
    }
  }
  if (owner && threadIdx.x == 0) owner[b] = who;
  if (who < 0) return;
  const int32_t slot = L - p * bs;
  auto store = [&](int32_t i, i32x4 val) {
    const int32_t h = i / per_head, j = i - h * per_head;
    const int64_t row = ((int64_t)blk * Hkv + h) * bs + slot;
    if (j < kc)
      k_cache[row * kc + j] = val;
    else
      v_cache[row * vc + (j - kc)] = val;
  };
  if (i0 < total) store(i0, first);
  for (int32_t i = i0 + kAppendThreads; i < total; i += kAppendThreads) store(i, src_of(i));
}

hipError_t launch_append_kv(const dcp_attn_shape& sh, const int32_t* seq_lens,
                            const void* new_k, const void* new_v, const int32_t* block_table,
                            void* k_cache, void* v_cache, int32_t* owner, hipStream_t stream) {
  const int32_t esize = sh.dtype == DCP_F32 ? 4 : 2;
  const bool gqa = sh.kv_kind == DCP_KV_GQA;
  const int32_t kc = sh.head_dim_qk * esize / 16;
  const int32_t vc = gqa ? sh.head_dim_v * esize / 16 : 0;
  hipLaunchKernelGGL(append_kv_kernel, dim3(sh.batch), dim3(kAppendThreads), 0, stream, seq_lens,
                     block_table, (const i32x4*)new_k, (const i32x4*)new_v, (i32x4*)k_cache,
                     (i32x4*)v_cache, owner, gqa ? sh.num_kv_heads : 1, kc, vc, sh.block_size,
                     sh.max_blocks_per_seq, sh.num_blocks, sh.num_shards);
  return hipGetLastError();
}

// ---------------------------------------------------------------- HBM read ceiling

// Measurement aid, not part of the attention path: stream a buffer with 128-bit non-temporal
// loads and fold the words so that the loads stay live. A workgroup reads 64 KB of
// consecutive bytes per iteration (eight 1 KB loads per wave, all in flight at once), and
// the workgroups take the 64 KB chunks in turn.
constexpr int kStreamThreads = 512;
constexpr int64_t kStreamChunk16 = 8 * kStreamThreads;  // 16-byte words per chunk (64 KB)

__global__ void __launch_bounds__(kStreamThreads)
stream_read_kernel(const u32x4* __restrict__ src, int64_t n16, int32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t acc = 0;
  for (int64_t c = (int64_t)blockIdx.x * kStreamChunk16; c < n16;
       c += (int64_t)gridDim.x * kStreamChunk16) {
    u32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int64_t i = c + 64 * (8 * k + wv) + lane;  // 1 KB block 8 k + wv of the chunk
      v[k] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  // one word per workgroup (lane 0 of wave 0), so the result is used
  if (threadIdx.x == 0) sink[blockIdx.x] = (int32_t)acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, int32_t* sink, int32_t blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kStreamThreads), 0, stream,
                     (const u32x4*)src, (int64_t)(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace dcp
