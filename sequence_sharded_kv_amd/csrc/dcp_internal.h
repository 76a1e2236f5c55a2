// Internal declarations shared by the host dispatcher and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dcp.h"

namespace dcp {

// Head region of the workspace: the flag word, then a row of zeros.
constexpr size_t kWsHeadBytes = 4096;
constexpr size_t kWsZeroOffset = 256;
constexpr int32_t kWsZeroWords = 512;  // 2 KB of zeros

// Flag bits in the workspace's sticky device flag word.
constexpr int32_t kFlagBoundClamped = 1;
constexpr int32_t kFlagBadBlock = 2;
constexpr int32_t kFlagRecomputed = 4;  // a worker's range was recomputed (see mla_pair16_kernel)
constexpr int32_t kFlagRescaled = 8;    // a worker raised a row's reference and rescaled it

// Work is split stream-K style: every (unit, page) pair is one page of work, the pages of
// all units are concatenated in unit order, and worker w takes the contiguous range
// [w*T/P, (w+1)*T/P). A unit is (request, shard, row group) for MLA and (request, shard,
// kv head, row group) for GQA. A unit cut by a worker boundary yields pieces (partials over
// sub-ranges) that a finishing pass merges into the unit's partial.
//
// Query rows: a request scores Tq query tokens (1 for plain decode) against its context;
// row rho = j * Hq + h is head h of query token j (R = Tq * Hq rows per request). The rows
// that read one KV head (its G heads of every token: G * Tq rows; MLA: G = Hq) are cut into
// groups of Ru rows, one unit each. Local row r of group rg is rr = rg * Ru + r of that
// space (rows with rr >= G * Tq are padding), i.e. token j = rr / G, head kvh * G + rr % G.
// Token j sits at position qend[b] + j, qend[b] = L_b - Tq with L_b the largest end among
// the request's ranges, and sees the context positions up to its own.
//
// Workspace layout (offsets 256-byte aligned):
//   flags      int32[64]  sticky device flag word at [0], the number of entries of `fin` at
//                         [1], then a 2 KB zero row at byte 256 (read in place of a page
//                         whose block id is invalid)
//   pre        int32[U + 1]      exclusive prefix sum of unit page counts, pre[U] = T
//   fin        int32[U][4]       units the finishing pass must write: (u, first worker, last
//                                worker, 0) for units cut by worker boundaries, (u, -1, -1, 0)
//                                for units with no pages; unordered
//   ubounds    int32[B*S*2]      sanitised (start, end) per (request, shard)
//   qend       int32[B]          position of each request's first query token
//   redo       int32[Pmax]       workers a kernel marked for recomputation
//   usrc       int32[U][4]       per unit, who wrote it: (first worker, last worker, piece slot
//                                of the first, first page); the two workers are equal for a
//                                unit written whole, -1 for a unit with no pages
//   piece_o    float[2*Pmax][Ru][Dv]
//   piece_lse  float[2*Pmax][Ru]
//   part_o     float[B][S][R][Dv]    (fused path only)
//   part_lse   float[B][S][R]
struct WsLayout {
  size_t flags, pre, fin, ubounds, qend, redo, usrc, piece_o, piece_lse, part_o, part_lse,
      total;
};

enum class Kernel { kNone = 0, kGqaValu, kGqaMfma, kGqaChunk, kMlaMfma };

struct Plan {          // host-side decisions for one shape
  Kernel kernel;
  int32_t units;           // U
  int32_t rows_per_unit;   // Ru
  int32_t row_groups;      // row groups per KV head
  int32_t max_workers;     // Pmax
  WsLayout ws;
};

// Parameters of the partial-attention kernels (passed by value).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* ubounds;   // [B*S][2]
  const int32_t* pre;       // [U + 1]
  const int32_t* fin;       // [U][4], count in flags[1]
  const int32_t* usrc;      // [U][4] writers of each unit
  const int32_t* qend;      // [B]
  float* part_o;            // [B][S][R][Dv]
  float* part_lse;          // [B][S][R]
  float* piece_o;           // [2P][Ru][Dv]
  float* piece_lse;         // [2P][Ru]
  int32_t* flags;
  int32_t* redo;            // [P] workers to recompute (cleared by the schedule kernel)
  const char* zero_row;     // kWsZeroWords*4 bytes of zeros in the workspace
  int32_t B, S, Hq, Hkv, G, Dqk, Dv, bs, max_blocks, num_blocks, U, P;
  int32_t Tq, R, Ru, NRg;   // query tokens, rows per request, rows per unit, groups per KV head
  // A call may run its query tokens in passes: this pass takes tokens j0 .. j0 + Tq - 1 of the
  // request's Tq_all, whose q, out and out_lse rows are Rs = Hq * Tq_all apart per request
  // (Rs = R and j0 = 0 for a single pass). Partial rows of (request, shard) bsi sit Rp rows
  // apart from row rp0 on: the caller's rows for the partial calls (Rp = Rs, rp0 = j0 * Hq),
  // the pass's own rows in the workspace for the fused calls (Rp = R, rp0 = 0).
  int32_t Rs, j0, Rp, rp0;
  float scale_log2;         // softmax_scale * log2(e)
};

// Row of the caller's q / out / out_lse for row rho of this pass of request b.
__host__ __device__ inline int64_t call_row(const AttnArgs& a, int32_t b, int32_t rho) {
  return (int64_t)b * a.Rs + (int64_t)a.j0 * a.Hq + rho;
}

// Row of part_o / part_lse for row rho of this pass of (request, shard) bsi.
__host__ __device__ inline int64_t part_row(const AttnArgs& a, int64_t bsi, int32_t rho) {
  return bsi * a.Rp + a.rp0 + rho;
}

// Query row of local row `r` of row group `rg` of KV head `kvh` (see "Query rows" above):
// returns rho, or -1 for a padding row; *j receives the query token.
__host__ __device__ inline int32_t unit_row(const AttnArgs& a, int32_t kvh, int32_t rg, int32_t r,
                                            int32_t* j) {
  const int32_t rr = rg * a.Ru + r;
  if (r >= a.Ru || rr >= a.G * a.Tq) return -1;
  *j = rr / a.G;
  return *j * a.Hq + kvh * a.G + (rr - *j * a.G);
}

// Launchers (each returns the hipError_t of its launch).
hipError_t launch_plan_device(const int32_t* seq_lens, int32_t B, int32_t S, int32_t bs,
                              int32_t* bounds, hipStream_t stream);
hipError_t launch_schedule(const int32_t* bounds, int32_t B, int32_t S, int32_t units_per_bs,
                           int32_t P, int32_t* fin,
                           int32_t bs, int32_t max_blocks, int32_t* ubounds, int32_t* pre,
                           int32_t* flags, int32_t Tq, int32_t* qend, int32_t* redo,
                           int32_t* usrc, int32_t keep_flags, hipStream_t stream);
hipError_t launch_finish_units(const AttnArgs& a, hipStream_t stream);
// out / out_lse straight from the pieces and partials (fused calls; no finishing pass)
hipError_t launch_combine(const AttnArgs& a, float* out, float* out_lse, hipStream_t stream);
hipError_t launch_merge(int32_t B, int32_t S, int32_t H, int32_t Dv, const float* part_o,
                        const float* part_lse, float* out, float* out_lse, hipStream_t stream);
hipError_t launch_debug_gather(const dcp_attn_shape& sh, const void* cache,
                               const int32_t* block_table, const int32_t* bounds, int32_t b,
                               int32_t s, int32_t kv_head, void* dst, int32_t max_rows,
                               hipStream_t stream);
hipError_t launch_append_kv(const dcp_attn_shape& sh, const int32_t* seq_lens,
                            const void* new_k, const void* new_v, const int32_t* block_table,
                            void* k_cache, void* v_cache, int32_t* owner, hipStream_t stream);

// Partial-attention kernels. `workers` returns the P the launcher will use (<= max_workers).
int32_t gqa_valu_workers(int device, int32_t max_workers);
hipError_t launch_gqa_valu(const AttnArgs& a, int32_t dtype, hipStream_t stream);
int32_t gqa_mfma_workers(int device, int32_t Dqk, int32_t max_workers);
hipError_t launch_gqa_mfma(const AttnArgs& a, hipStream_t stream);
int32_t gqa_chunk_workers(int device, int32_t Ru, int32_t max_workers);
hipError_t launch_gqa_chunk(const AttnArgs& a, hipStream_t stream);
int32_t mla_mfma_workers(int device, int32_t Ru, int32_t max_workers);
hipError_t launch_mla_mfma(const AttnArgs& a, hipStream_t stream);
hipError_t launch_mla_ring(const AttnArgs& a, hipStream_t stream);  // 64 rows per unit
hipError_t launch_mla_pair16(const AttnArgs& a, hipStream_t stream);  // 128 rows per unit
hipError_t launch_stream_read(const void* src, size_t bytes, int32_t* sink, int32_t blocks,
                              hipStream_t stream);

}  // namespace dcp
