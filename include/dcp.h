/*
 * dcp.h -- sequence-sharded paged decode attention for MI355X (gfx950).
 *
 * The operation is the decode-time step of Decode Context Parallelism:
 *
 *  1. The KV cache of each request is split along the sequence into
 *     contiguous token shards [start, end); each DCP rank owns one range
 *     (Qiita article on vLLM -dcp, section on assigning token ranges to GPUs;
 *     naphjohn blog "Inference Systems Infrastructure Notes (7)", section 2).
 *  2. The one-token decode query attends over each shard's KV only, giving a
 *     partial result: the shard's softmax output O_s and its log-sum-exp
 *     LSE_s (same Qiita section, second step of its three).
 *  3. The partials are combined by online-softmax re-weighting into exactly
 *     the attention over the whole context (same Qiita section, third step;
 *     blog section 2):  M = max_s LSE_s,  LSE = M + ln sum_s exp(LSE_s - M),
 *     O = sum_s exp(LSE_s - LSE) * O_s.
 *  4. The intermediate partials live in one caller-owned workspace that is
 *     reused every step instead of being allocated per call (blog section 3,
 *     scratch-buffer reuse).
 *
 * On one GPU every shard of every request is resident; the shards stand in
 * for the ranks of a DCP group and no collective is issued.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every entry point returns a dcp_status. Host-checkable problems (NULL
 *    or misaligned pointers, sizes, unsupported shapes, workspace too small)
 *    are reported before any device work is queued. Nothing throws across
 *    this ABI. dcp_last_error() returns a thread-local detail string for the
 *    last failing call on the calling thread.
 *  - Device entry points queue kernels on `stream` (a hipStream_t passed as
 *    void*; NULL means the legacy default stream) and never synchronise.
 *  - All memory is owned by the caller. The library allocates no device
 *    memory and keeps no state beyond a per-device cache of launch
 *    parameters, the thread-local error string and, between
 *    dcp_kernel_timing_begin and _end, the calling thread's timing events.
 *    The one exception is the static device scratch of
 *    dcp_decode_attn_noalloc (DCP_NOALLOC_SCRATCH_BYTES per GPU, part of the
 *    loaded module and held until the process ends).
 *  - Device pointers to Q, caches, partials, outputs and workspace must be
 *    16-byte aligned (the kernels use 128-bit loads and stores).
 *  - Values that only exist on the device (bounds, block-table entries) are
 *    checked by the kernels without faulting: a bound outside
 *    [0, max_blocks_per_seq * block_size] is clamped, a block id outside
 *    [0, num_blocks) is treated as a page of masked tokens, and either event
 *    sets a sticky bit in the workspace (dcp_read_device_flags).
 */
#ifndef DCP_H_
#define DCP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCP_ABI_VERSION 1

typedef int32_t dcp_status;
enum {
  DCP_OK = 0,
  DCP_ERR_NULL = 1,        /* a required pointer is NULL */
  DCP_ERR_SHAPE = 2,       /* sizes out of range or inconsistent */
  DCP_ERR_UNSUPPORTED = 3, /* valid request that no kernel implements */
  DCP_ERR_WORKSPACE = 4,   /* workspace smaller than dcp_workspace_bytes() */
  DCP_ERR_BAD_PLAN = 5,    /* host-visible sequence lengths are invalid (negative) */
  DCP_ERR_ALIGN = 6,       /* a device pointer is not 16-byte aligned */
  DCP_ERR_DEVICE = 7       /* the HIP runtime reported an error */
};

/* Element type of Q and of the KV cache (both the same). */
enum { DCP_F32 = 0, DCP_BF16 = 1 };

/* Cache layout.
 * DCP_KV_GQA: separate K and V caches, each [num_blocks][num_kv_heads][block_size][head_dim]
 *             (one KV head of one page is a contiguous block_size x head_dim tile).
 *             head_dim_qk == head_dim_v. Query head h reads KV head h / (num_q_heads / num_kv_heads).
 * DCP_KV_MLA: one latent cache [num_blocks][block_size][head_dim_qk] shared by all query heads
 *             (num_kv_heads == 1); the value of a token is the first head_dim_v entries of its
 *             cached row (absorbed MLA: 576 = 512 latent + 64 rope, value 512). v_cache is NULL.
 * Token t of request b is in page block_table[b * max_blocks_per_seq + t / block_size], at slot
 * t % block_size (paged KV, vLLM's PagedAttention blocks). */
enum { DCP_KV_GQA = 0, DCP_KV_MLA = 1 };

typedef struct dcp_attn_shape {
  int32_t batch;              /* B >= 1 requests, one decode query token each */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv; Hq % Hkv == 0; 1 for MLA */
  int32_t head_dim_qk;        /* Dqk: dims of q and k */
  int32_t head_dim_v;         /* Dv: dims of v and of the output */
  int32_t block_size;         /* tokens per KV page */
  int32_t max_blocks_per_seq; /* row length of block_table */
  int32_t num_blocks;         /* pages in the cache pool */
  int32_t num_shards;         /* S shards per request */
  int32_t dtype;              /* DCP_F32 or DCP_BF16, for q and caches */
  int32_t kv_kind;            /* DCP_KV_GQA or DCP_KV_MLA */
  float softmax_scale;        /* scores are softmax_scale * <q, k> */
} dcp_attn_shape;

/* DCP_ABI_VERSION of the loaded library. */
int32_t dcp_abi_version(void);

/* Static description of a status code (never NULL). */
const char* dcp_status_string(dcp_status status);

/* Detail of the last failing call on this thread ("" if none). */
const char* dcp_last_error(void);

/*
 * dcp_plan_shards -- host only, no device work.
 * The canonical split of each request into num_shards contiguous token ranges that start on
 * page boundaries (Qiita section on token ranges: 200K tokens over 4 ranks gives 0-50K,
 * 50K-100K, ...). With P = ceil(L / block_size) pages and k = ceil(P / num_shards):
 *   start_s = min(L, s*k*block_size),  end_s = min(L, (s+1)*k*block_size).
 * The last non-empty shard may be ragged; trailing shards may be empty (start == end == L).
 *   seq_lens: host int32[batch], each >= 0 (negative -> DCP_ERR_BAD_PLAN).
 *   bounds:   host int32[batch][num_shards][2] written as (start, end).
 * Errors: DCP_ERR_NULL, DCP_ERR_SHAPE (batch < 1, num_shards < 1, block_size < 1),
 * DCP_ERR_BAD_PLAN. Nothing is written on error.
 */
dcp_status dcp_plan_shards(const int32_t* seq_lens, int32_t batch, int32_t num_shards,
                           int32_t block_size, int32_t* bounds);

/*
 * dcp_plan_shards_device -- the same plan computed on the device from device seq_lens
 * (int32[batch]) into device bounds (int32[batch][num_shards][2]). Negative lengths are
 * treated as 0. Asynchronous on `stream`.
 */
dcp_status dcp_plan_shards_device(const int32_t* seq_lens, int32_t batch, int32_t num_shards,
                                  int32_t block_size, int32_t* bounds, void* stream);

/*
 * dcp_workspace_bytes -- host only. Size of the workspace that dcp_decode_attn_partial and
 * dcp_decode_attn need for this shape (the larger, fused, requirement). Allocate it once for
 * the largest shape in use and pass it to every call. Errors: DCP_ERR_NULL, DCP_ERR_SHAPE,
 * DCP_ERR_UNSUPPORTED.
 */
dcp_status dcp_workspace_bytes(const dcp_attn_shape* shape, size_t* bytes);

/*
 * dcp_decode_attn_partial -- step 2: per-shard partial attention.
 *   q:           device [B][Hq][Dqk] (dtype)
 *   k_cache:     device, GQA [num_blocks][Hkv][block_size][Dqk]; MLA [num_blocks][block_size][Dqk]
 *   v_cache:     device, GQA same layout as k_cache (Dv == Dqk); MLA must be NULL
 *   block_table: device int32 [B][max_blocks_per_seq]
 *   bounds:      device int32 [B][S][2]: shard s of request b covers tokens [start, end).
 *                Any ranges are accepted (the canonical plan or any other); the merge gives
 *                the full attention when they partition [0, L_b).
 *   part_o:      device float [B][S][Hq][Dv]: O_s (softmax output over the shard, fp32)
 *   part_lse:    device float [B][S][Hq]: LSE_s = ln sum_{t in shard} exp(scale*<q,k_t>);
 *                an empty shard gives O_s = 0 and LSE_s = -inf.
 *   workspace:   device, >= dcp_workspace_bytes(); its content need not be initialised
 *                and is overwritten (do not share one workspace between concurrent calls).
 * Errors: DCP_ERR_NULL, DCP_ERR_ALIGN, DCP_ERR_SHAPE, DCP_ERR_UNSUPPORTED,
 * DCP_ERR_WORKSPACE, DCP_ERR_DEVICE.
 */
dcp_status dcp_decode_attn_partial(const dcp_attn_shape* shape, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* bounds,
                                   float* part_o, float* part_lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * dcp_merge_lse -- step 3: combine S partials per (request, head) by LSE re-weighting.
 *   part_o [B][S][H][Dv], part_lse [B][S][H] (device float) -> out [B][H][Dv] (device float)
 *   and, if out_lse is not NULL, out_lse [B][H] = the log-sum-exp over the union of shards.
 * Shards with LSE = -inf contribute nothing; if all are -inf, out = 0 and out_lse = -inf.
 * Errors: DCP_ERR_NULL, DCP_ERR_ALIGN, DCP_ERR_SHAPE, DCP_ERR_DEVICE.
 */
dcp_status dcp_merge_lse(int32_t batch, int32_t num_shards, int32_t num_heads, int32_t head_dim_v,
                         const float* part_o, const float* part_lse, float* out, float* out_lse,
                         void* stream);

/*
 * dcp_decode_attn -- steps 2 and 3 in one call: the per-shard partials are kept in the
 * workspace (reused every call, step 4) and merged into out [B][Hq][Dv] (device float) and,
 * if not NULL, out_lse [B][Hq]. Arguments as for dcp_decode_attn_partial.
 */
dcp_status dcp_decode_attn(const dcp_attn_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table, const int32_t* bounds,
                           void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                           void* stream);

/*
 * dcp_decode_attn_noalloc -- dcp_decode_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * workspace is a device array inside the library, DCP_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU,
 * one copy on each GPU the library runs on, kept until the process ends. Arguments, results
 * and errors are those of dcp_decode_attn without the workspace pair. The call allocates
 * nothing: no hipMalloc, hipFree or allocating library routine (the first call on a device
 * looks up that device's copy of the array once). Every call on one GPU shares that GPU's
 * scratch, which keeps the last call's contents; each call rewrites all it reads before
 * reading it, so no clearing is needed, but calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race on it and give undefined results.
 * Errors additionally: DCP_ERR_WORKSPACE, before any device work, when the shape needs more
 * than DCP_NOALLOC_SCRATCH_BYTES of workspace (dcp_workspace_bytes); DCP_ERR_DEVICE when the
 * current device index is 64 or above.
 */
#define DCP_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
dcp_status dcp_decode_attn_noalloc(const dcp_attn_shape* shape, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* bounds, float* out,
                                   float* out_lse, void* stream);

/*
 * Several query tokens per request: speculative decoding / MTP verification (2 .. 16 tokens)
 * and chunked or cached prefill (a chunk of up to 4096 tokens). Both pages name speculative
 * decoding and MTP as what DCP is to be combined with (Qiita article, section on how to view
 * it in practice; naphjohn blog, section 5), and the blog's section 4 has DCP reach chunked
 * prefill (long inputs prefilled chunk by chunk) and cached prefill (reusing KV already
 * computed). A call scores the q_len newest tokens of each request at once, against the
 * sharded cache that already holds their K/V: query token j of request b sits at position
 * L_b - q_len + j, where L_b is the largest end among b's ranges in `bounds`, its K/V is
 * already in the cache, and it sees the positions up to and including its own (causal
 * order). The shards, the partials and the merge are as for one token; a row that sees
 * nothing in a shard gets O_s = 0, LSE_s = -inf, and one that sees nothing at all (L_b <
 * q_len - j) gets O = 0, LSE = -inf. q_len = 1 is exactly dcp_decode_attn[_partial].
 *   q_len:     1 .. 4096 query tokens per request.
 *   q:         device [B][q_len][Hq][Dqk] (dtype).
 *   part_o:    device float [B][S][q_len][Hq][Dv];  part_lse: device float [B][S][q_len][Hq].
 *   out:       device float [B][q_len][Hq][Dv];     out_lse:  device float [B][q_len][Hq] or NULL.
 *   The other arguments, the workspace rules and the errors are those of the one-token calls;
 *   the workspace must hold dcp_workspace_bytes_multi(shape, q_len) bytes. dcp_merge_lse merges
 *   these partials when called with num_heads = q_len * Hq.
 * The KV pages are streamed once per group of query rows that share them: MLA takes up to 128
 * rows (q_len * Hq) in one pass, GQA up to 256 rows (q_len * Hq / Hkv) per KV head for bf16
 * head dim 128 and 16 for the other GQA shapes; a prefill
 * chunk therefore streams each shard's pages once per row group, as a flash-attention query
 * block does. MLA calls of 129 to 192 rows stream the pages twice: the first 128 rows and the
 * remaining tokens run as two passes over the same workspace, one after the other on the
 * stream, each writing its own rows of the outputs. The fused call keeps B * S * q_len * Hq
 * partials in the workspace (those of one pass at a time). Errors
 * additionally: DCP_ERR_SHAPE for q_len outside [1, 4096].
 */
dcp_status dcp_workspace_bytes_multi(const dcp_attn_shape* shape, int32_t q_len, size_t* bytes);
dcp_status dcp_decode_attn_multi_partial(const dcp_attn_shape* shape, int32_t q_len,
                                         const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* bounds,
                                         float* part_o, float* part_lse, void* workspace,
                                         size_t workspace_bytes, void* stream);
dcp_status dcp_decode_attn_multi(const dcp_attn_shape* shape, int32_t q_len, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* bounds,
                                 void* workspace, size_t workspace_bytes, float* out,
                                 float* out_lse, void* stream);

/*
 * dcp_read_device_flags -- copy the sticky device-side flag word out of a workspace and
 * wait for `stream`. Bit 0: a bound was clamped into [0, max_blocks_per_seq*block_size] or
 * had end < start. Bit 1: a block id outside [0, num_blocks) was met and its tokens masked.
 * Bit 2 (informational, results unaffected): on the MLA path with 128 query rows per unit,
 * whose value product runs in fp16, a worker met a latent value of magnitude 65504 or more, or
 * a segment whose nonzero values all stay below 2^-10, and its range was recomputed in bf16 by
 * the general kernel. Bit 3 (informational, results unaffected): on the MLA paths with 64 or
 * 128 query rows per unit or on the GQA bf16 head-dim-128 path, a tile's scores exceeded a
 * row's reference (the maximum of its first tile with a visible token) by more than the
 * weights' margin, and the row's reference was raised and its sum and accumulator rescaled in
 * place. Bits are cleared by the next attention call on that workspace; a fused call that
 * runs in two passes reports the bits of both.
 */
dcp_status dcp_read_device_flags(const void* workspace, int32_t* flags, void* stream);

/*
 * dcp_debug_gather_shard -- test aid for bit-exact page indexing. Copies the cached rows of
 * tokens [start, end) of shard (b, s) (bounds read on the device, clamped as above) for KV
 * head kv_head (GQA; 0 for MLA) from `cache` into dst, row after row, as raw element bits
 * (head_dim_qk elements per row of the cache's dtype). At most max_rows rows are written.
 */
dcp_status dcp_debug_gather_shard(const dcp_attn_shape* shape, const void* cache,
                                  const int32_t* block_table, const int32_t* bounds, int32_t b,
                                  int32_t s, int32_t kv_head, void* dst, int32_t max_rows,
                                  void* stream);

/*
 * dcp_append_kv -- the step that precedes attention on every decode step: store the K/V (GQA)
 * or latent (MLA) row of the token each request just produced. Decode emits one token per
 * request per step and, under DCP, only the rank owning the token's range keeps its KV
 * (naphjohn blog "Inference Systems Infrastructure Notes (7)", section 4, decode bullet;
 * Qiita article on vLLM -dcp, section on assigning token ranges to GPUs). A request that
 * holds L_b tokens stores its new token at position L_b: slot L_b % block_size of page
 * block_table[b * max_blocks_per_seq + L_b / block_size] (paged KV, as for attention).
 *   shape:       as for attention; batch, num_kv_heads, head_dim_qk, head_dim_v, block_size,
 *                max_blocks_per_seq, num_blocks, num_shards, dtype and kv_kind are used.
 *   seq_lens:    device int32 [B]: L_b, tokens cached before this step (the new position).
 *   new_k:       device, GQA [B][Hkv][Dqk]; MLA [B][Dqk] (the latent row, rope part included).
 *   new_v:       device, GQA [B][Hkv][Dv]; MLA must be NULL.
 *   block_table: device int32 [B][max_blocks_per_seq].
 *   k_cache, v_cache: device caches in the attention layouts, updated in place (v_cache NULL
 *                for MLA). Only the B addressed rows (per KV head) are written.
 *   owner:       device int32 [B] or NULL. owner[b] = the shard whose range in the canonical
 *                plan of L_b + 1 tokens (dcp_plan_shards) holds position L_b, i.e. the last
 *                non-empty shard; -1 if L_b < 0 or L_b / block_size >= max_blocks_per_seq;
 *                -2 if the table entry is outside [0, num_blocks). Nothing is stored for a
 *                request with a negative owner.
 * Row bytes (Dqk, and Dv for GQA, times the element size) must be multiples of 16. The new
 * rows must not overlap the caches, and two requests must not address the same (page, slot)
 * in one call (which of them is kept is then unspecified). Asynchronous on `stream`.
 * Errors: DCP_ERR_NULL, DCP_ERR_ALIGN, DCP_ERR_SHAPE (also: MLA with new_v or v_cache),
 * DCP_ERR_UNSUPPORTED (row bytes), DCP_ERR_DEVICE.
 */
dcp_status dcp_append_kv(const dcp_attn_shape* shape, const int32_t* seq_lens, const void* new_k,
                         const void* new_v, const int32_t* block_table, void* k_cache,
                         void* v_cache, int32_t* owner, void* stream);

/*
 * dcp_hbm_read_ceiling -- measurement aid, not part of the attention path: read `bytes` (a
 * positive multiple of 16) of the device buffer `src` (16-byte aligned) once with 128-bit
 * non-temporal loads spread over every CU, and write one word per workgroup to `sink`
 * (device int32, at least 2 x the CU count entries; the values are meaningless). Timing a few
 * launches over a buffer of some GiB gives the HBM read rate that a plain streaming kernel
 * reaches on this device, which bench.py reports beside the 8 TB/s peak. Errors: DCP_ERR_NULL,
 * DCP_ERR_ALIGN, DCP_ERR_SHAPE, DCP_ERR_DEVICE.
 */
dcp_status dcp_hbm_read_ceiling(const void* src, size_t bytes, int32_t* sink, void* stream);

/*
 * Kernel timing for benchmarks (no effect on results). dcp_kernel_timing_begin(n) creates n
 * pairs of HIP events; while timing is on for the calling thread, each of the next n
 * dcp_decode_attn / dcp_decode_attn_partial calls records one pair around its
 * partial-attention kernel, on the call's stream. dcp_kernel_timing_end() waits for the
 * recorded events, returns how many launches were timed and their summed duration in
 * milliseconds, and releases the events. Errors: DCP_ERR_SHAPE (n < 1), DCP_ERR_NULL,
 * DCP_ERR_DEVICE.
 */
dcp_status dcp_kernel_timing_begin(int32_t max_launches);
dcp_status dcp_kernel_timing_end(int32_t* launches, float* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DCP_H_ */
