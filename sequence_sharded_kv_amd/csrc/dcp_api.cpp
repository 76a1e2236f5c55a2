// Host side of the C ABI: argument validation, the shard plan, kernel choice, workspace
// layout and the launch sequence. Every device entry point queues its kernels on the
// caller's stream and returns without synchronising.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dcp_internal.h"

namespace {

thread_local std::string g_last_error;

// Benchmark timing: pre-created event pairs, filled one per timed launch.
struct KernelTiming {
  std::vector<hipEvent_t> start, stop;
  size_t used = 0;
  bool on = false;
};
thread_local KernelTiming g_timing;

void destroy_timing_events() {
  for (hipEvent_t e : g_timing.start) (void)hipEventDestroy(e);
  for (hipEvent_t e : g_timing.stop) (void)hipEventDestroy(e);
  g_timing.start.clear();
  g_timing.stop.clear();
  g_timing.used = 0;
  g_timing.on = false;
}

dcp_status fail(dcp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dcp_status ok() {
  g_last_error.clear();
  return DCP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Workspace of dcp_decode_attn_noalloc: a file-scope device array, one copy per GPU, held
// from the module's load until the process ends. Its name is a host-side stand-in; kernels
// get the device address that hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) char scratch[DCP_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Upper bounds on workers (stream-K ranges) per kernel family; the launch uses at most this.
constexpr int32_t kMaxWorkersWave = 4096;  // GQA kernels: one wave per worker
constexpr int32_t kMaxWorkersMla = 512;    // MLA kernel: one workgroup per worker
constexpr int32_t kMaxWorkersChunk = 1024; // GQA chunk kernel: one workgroup per worker

dcp_status check_shape(const dcp_attn_shape* sh) {
  if (!sh) return fail(DCP_ERR_NULL, "shape is NULL");
  if (sh->batch < 1 || sh->num_q_heads < 1 || sh->num_kv_heads < 1 || sh->head_dim_qk < 1 ||
      sh->head_dim_v < 1 || sh->block_size < 1 || sh->max_blocks_per_seq < 1 ||
      sh->num_blocks < 1 || sh->num_shards < 1)
    return fail(DCP_ERR_SHAPE, "every size must be >= 1 (batch=%d Hq=%d Hkv=%d Dqk=%d Dv=%d "
                "bs=%d max_blocks=%d num_blocks=%d S=%d)", sh->batch, sh->num_q_heads,
                sh->num_kv_heads, sh->head_dim_qk, sh->head_dim_v, sh->block_size,
                sh->max_blocks_per_seq, sh->num_blocks, sh->num_shards);
  if (sh->num_q_heads % sh->num_kv_heads != 0)
    return fail(DCP_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d",
                sh->num_q_heads, sh->num_kv_heads);
  if (sh->dtype != DCP_F32 && sh->dtype != DCP_BF16)
    return fail(DCP_ERR_SHAPE, "dtype %d is neither DCP_F32 nor DCP_BF16", sh->dtype);
  if (sh->kv_kind != DCP_KV_GQA && sh->kv_kind != DCP_KV_MLA)
    return fail(DCP_ERR_SHAPE, "kv_kind %d is neither DCP_KV_GQA nor DCP_KV_MLA", sh->kv_kind);
  if (!std::isfinite(sh->softmax_scale))
    return fail(DCP_ERR_SHAPE, "softmax_scale is not finite");
  if (sh->kv_kind == DCP_KV_GQA && sh->head_dim_v != sh->head_dim_qk)
    return fail(DCP_ERR_SHAPE, "GQA needs head_dim_v == head_dim_qk (%d != %d)", sh->head_dim_v,
                sh->head_dim_qk);
  if (sh->kv_kind == DCP_KV_MLA && (sh->num_kv_heads != 1 || sh->head_dim_v > sh->head_dim_qk))
    return fail(DCP_ERR_SHAPE, "MLA needs num_kv_heads == 1 and head_dim_v <= head_dim_qk");
  if (sh->head_dim_v % 4 != 0)
    return fail(DCP_ERR_SHAPE, "head_dim_v %d is not a multiple of 4", sh->head_dim_v);
  const int64_t units = (int64_t)sh->batch * sh->num_shards *
                        (sh->kv_kind == DCP_KV_GQA ? sh->num_kv_heads : 1);
  if ((int64_t)sh->max_blocks_per_seq * sh->block_size > INT32_MAX)
    return fail(DCP_ERR_SHAPE, "max_blocks_per_seq * block_size exceeds int32");
  if (units * (int64_t)sh->max_blocks_per_seq > INT32_MAX)
    return fail(DCP_ERR_SHAPE, "batch * num_shards * kv units * max_blocks_per_seq exceeds int32");
  if ((int64_t)sh->batch * sh->num_shards > (1 << 24))
    return fail(DCP_ERR_SHAPE, "batch * num_shards exceeds 2^24");
  return DCP_OK;
}

// Most query tokens per request that the multi-token entry points take (a prefill chunk).
constexpr int32_t kMaxQueryTokens = 4096;

dcp_status make_plan(const dcp_attn_shape* sh, int32_t Tq, dcp::Plan* plan) {
  dcp_status st = check_shape(sh);
  if (st != DCP_OK) return st;
  if (Tq < 1 || Tq > kMaxQueryTokens)
    return fail(DCP_ERR_SHAPE, "q_len %d outside [1, %d]", Tq, kMaxQueryTokens);
  using dcp::Kernel;
  Kernel k = Kernel::kNone;
  int32_t ru, pmax;
  const int32_t G = sh->num_q_heads / sh->num_kv_heads;
  const int32_t rows = G * Tq;  // rows that read one KV head
  if (sh->kv_kind == DCP_KV_GQA) {
    const int32_t D = sh->head_dim_qk;
    if (sh->dtype == DCP_BF16 && G <= 16 && D == 128) {
      // units of 32 to 256 rows share each K/V tile (fewer rows are padded to 32: the
      // 32-row kernel streams a head's pages faster than the 16-row one even half empty)
      k = Kernel::kGqaChunk;
      ru = 32;
      while (ru < rows && ru < 256) ru *= 2;
      pmax = kMaxWorkersChunk;
    } else {
      if (sh->dtype == DCP_BF16 && G <= 16 && (D == 64 || D == 128))
        k = Kernel::kGqaMfma;
      else if (G <= 16 && D % 64 == 0 && D <= 256)
        k = Kernel::kGqaValu;
      ru = rows < 16 ? rows : 16;  // one 16-column MFMA block (or 16 VALU rows) per unit
      pmax = kMaxWorkersWave;
    }
  } else {
    if (sh->dtype == DCP_BF16 && sh->head_dim_qk == 576 && sh->head_dim_v == 512 &&
        (sh->num_q_heads == 16 || sh->num_q_heads == 32 || sh->num_q_heads == 64 ||
         sh->num_q_heads == 128))
      k = Kernel::kMlaMfma;
    // waves of 16 rows, a power of two of them up to 8 per workgroup
    ru = 16;
    while (ru < rows && ru < 128) ru *= 2;
    // 129 to 192 rows: the calls run two passes (split_tokens); this single-pass plan of
    // three 64-row units only enters the workspace size
    if (rows > 128 && rows <= 192) ru = 64;
    // units of 64 or 128 rows run one workgroup per CU (256 on gfx950), smaller ones two
    pmax = ru >= 64 ? kMaxWorkersMla / 2 : kMaxWorkersMla;
  }
  const int32_t groups = (rows + ru - 1) / ru;
  const int64_t units64 = (int64_t)sh->batch * sh->num_shards *
                          (sh->kv_kind == DCP_KV_GQA ? sh->num_kv_heads : 1) * groups;
  if (units64 * (int64_t)sh->max_blocks_per_seq > INT32_MAX)
    return fail(DCP_ERR_SHAPE, "units (%lld) * max_blocks_per_seq exceeds int32",
                (long long)units64);
  const int32_t units = (int32_t)units64;
  if (k == Kernel::kNone)
    return fail(DCP_ERR_UNSUPPORTED,
                "no kernel for kv_kind=%d dtype=%d Hq=%d Hkv=%d Dqk=%d Dv=%d (GQA: group <= 16, "
                "bf16 head_dim 64/128 or any dtype head_dim a multiple of 64 up to 256; MLA: bf16, "
                "576/512, 16/32/64/128 heads)",
                sh->kv_kind, sh->dtype, sh->num_q_heads, sh->num_kv_heads, sh->head_dim_qk,
                sh->head_dim_v);
  plan->kernel = k;
  plan->units = units;
  plan->rows_per_unit = ru;
  plan->row_groups = groups;
  plan->max_workers = pmax;
  dcp::WsLayout& w = plan->ws;
  const size_t B = sh->batch, S = sh->num_shards, R = (size_t)sh->num_q_heads * Tq;
  const size_t Dv = sh->head_dim_v;
  size_t off = 0;
  w.flags = off;       off = align_up(off + dcp::kWsHeadBytes);
  w.pre = off;         off = align_up(off + sizeof(int32_t) * ((size_t)units + 1));
  w.fin = off;         off = align_up(off + sizeof(int32_t) * 4 * (size_t)units);
  w.ubounds = off;     off = align_up(off + sizeof(int32_t) * B * S * 2);
  w.qend = off;        off = align_up(off + sizeof(int32_t) * B);
  w.redo = off;        off = align_up(off + sizeof(int32_t) * (size_t)pmax);
  w.usrc = off;        off = align_up(off + sizeof(int32_t) * 4 * (size_t)units);
  w.piece_o = off;     off = align_up(off + sizeof(float) * 2 * (size_t)pmax * ru * Dv);
  w.piece_lse = off;   off = align_up(off + sizeof(float) * 2 * (size_t)pmax * ru);
  w.part_o = off;      off = align_up(off + sizeof(float) * B * S * R * Dv);
  w.part_lse = off;    off = align_up(off + sizeof(float) * B * S * R);
  w.total = off;
  return DCP_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

dcp_status device_fail(hipError_t e, const char* what) {
  return fail(DCP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// MLA calls of 129 to 192 query rows run in two passes over the KV: the first 128 rows
// (128 / Hq tokens) as one 128-row unit, the remaining tokens as one unit of at most 64 rows.
// Returns the first pass's token count, or 0 where the call runs in one pass.
int32_t split_tokens(const dcp_attn_shape* sh, int32_t Tq) {
  if (sh->kv_kind != DCP_KV_MLA) return 0;
  const int64_t Hq = sh->num_q_heads, rows = Hq * Tq;
  return (rows > 128 && rows <= 192 && Hq <= 64 && 128 % Hq == 0) ? (int32_t)(128 / Hq) : 0;
}

// Shared front half of the two attention entry points: the partials of query tokens
// j0 .. j0 + Tq - 1 of a call with Tq_all tokens (j0 = 0, Tq_all = Tq for a single pass).
dcp_status run_partials(const dcp_attn_shape* sh, int32_t Tq, const void* q, const void* k,
                        const void* v, const int32_t* block_table, const int32_t* bounds,
                        float* part_o, float* part_lse, void* workspace, size_t workspace_bytes,
                        void* stream, dcp::Plan* plan_out, dcp::AttnArgs* args_out, bool fused,
                        int32_t j0 = 0, int32_t Tq_all = 0) {
  if (Tq_all == 0) Tq_all = Tq;
  dcp::Plan plan;
  dcp_status st = make_plan(sh, Tq, &plan);
  if (st != DCP_OK) return st;
  if (!q || !k || !block_table || !bounds || !workspace || (!fused && (!part_o || !part_lse)))
    return fail(DCP_ERR_NULL, "q, k_cache, block_table, bounds, workspace%s must be non-NULL",
                fused ? "" : ", part_o, part_lse");
  if (sh->kv_kind == DCP_KV_GQA && !v) return fail(DCP_ERR_NULL, "GQA needs v_cache");
  if (sh->kv_kind == DCP_KV_MLA && v)
    return fail(DCP_ERR_SHAPE, "MLA reads V from the latent cache; v_cache must be NULL");
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || !aligned16(workspace) ||
      (!fused && (!aligned16(part_o) || !aligned16(part_lse))))
    return fail(DCP_ERR_ALIGN, "q, caches, partials and workspace must be 16-byte aligned");
  if (workspace_bytes < plan.ws.total)
    return fail(DCP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes,
                plan.ws.total);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  char* ws = static_cast<char*>(workspace);
  dcp::AttnArgs a;
  memset(&a, 0, sizeof a);
  a.q = q;
  a.k = k;
  a.v = v;
  a.block_table = block_table;
  a.ubounds = reinterpret_cast<int32_t*>(ws + plan.ws.ubounds);
  a.pre = reinterpret_cast<int32_t*>(ws + plan.ws.pre);
  a.fin = reinterpret_cast<int32_t*>(ws + plan.ws.fin);
  a.usrc = reinterpret_cast<int32_t*>(ws + plan.ws.usrc);
  a.qend = reinterpret_cast<int32_t*>(ws + plan.ws.qend);
  a.redo = reinterpret_cast<int32_t*>(ws + plan.ws.redo);
  a.part_o = fused ? reinterpret_cast<float*>(ws + plan.ws.part_o) : part_o;
  a.part_lse = fused ? reinterpret_cast<float*>(ws + plan.ws.part_lse) : part_lse;
  a.piece_o = reinterpret_cast<float*>(ws + plan.ws.piece_o);
  a.piece_lse = reinterpret_cast<float*>(ws + plan.ws.piece_lse);
  a.flags = reinterpret_cast<int32_t*>(ws + plan.ws.flags);
  a.zero_row = ws + plan.ws.flags + dcp::kWsZeroOffset;
  a.B = sh->batch;
  a.S = sh->num_shards;
  a.Hq = sh->num_q_heads;
  a.Hkv = sh->num_kv_heads;
  a.G = sh->num_q_heads / sh->num_kv_heads;
  a.Dqk = sh->head_dim_qk;
  a.Dv = sh->head_dim_v;
  a.bs = sh->block_size;
  a.max_blocks = sh->max_blocks_per_seq;
  a.num_blocks = sh->num_blocks;
  a.U = plan.units;
  a.Tq = Tq;
  a.R = sh->num_q_heads * Tq;
  a.Rs = sh->num_q_heads * Tq_all;
  a.j0 = j0;
  a.Rp = fused ? a.R : a.Rs;  // the fused calls keep each pass's partials in the workspace
  a.rp0 = fused ? 0 : j0 * sh->num_q_heads;
  a.Ru = plan.rows_per_unit;
  a.NRg = plan.row_groups;
  a.scale_log2 = sh->softmax_scale * 1.4426950408889634f;
  switch (plan.kernel) {
    case dcp::Kernel::kGqaMfma: a.P = dcp::gqa_mfma_workers(dev, a.Dqk, plan.max_workers); break;
    case dcp::Kernel::kGqaValu: a.P = dcp::gqa_valu_workers(dev, plan.max_workers); break;
    case dcp::Kernel::kGqaChunk: a.P = dcp::gqa_chunk_workers(dev, a.Ru, plan.max_workers); break;
    case dcp::Kernel::kMlaMfma: a.P = dcp::mla_mfma_workers(dev, a.Ru, plan.max_workers); break;
    default: return fail(DCP_ERR_UNSUPPORTED, "no kernel");
  }
  hipStream_t s = as_stream(stream);
  const int32_t units_per_bs = plan.units / (sh->batch * sh->num_shards);
  e = dcp::launch_schedule(bounds, a.B, a.S, units_per_bs, a.P,
                           reinterpret_cast<int32_t*>(ws + plan.ws.fin), a.bs, a.max_blocks,
                           const_cast<int32_t*>(a.ubounds), const_cast<int32_t*>(a.pre), a.flags,
                           Tq_all, const_cast<int32_t*>(a.qend), a.redo,
                           const_cast<int32_t*>(a.usrc), j0 > 0 ? 1 : 0, s);
  if (e != hipSuccess) return device_fail(e, "schedule launch");
  const bool timed = g_timing.on && g_timing.used < g_timing.start.size();
  if (timed) {
    e = hipEventRecord(g_timing.start[g_timing.used], s);
    if (e != hipSuccess) return device_fail(e, "timing event");
  }
  switch (plan.kernel) {
    case dcp::Kernel::kGqaMfma: e = dcp::launch_gqa_mfma(a, s); break;
    case dcp::Kernel::kGqaValu: e = dcp::launch_gqa_valu(a, sh->dtype, s); break;
    case dcp::Kernel::kGqaChunk: e = dcp::launch_gqa_chunk(a, s); break;
    case dcp::Kernel::kMlaMfma: e = dcp::launch_mla_mfma(a, s); break;
    default: break;
  }
  if (e != hipSuccess) return device_fail(e, "partial-attention launch");
  if (timed) {
    e = hipEventRecord(g_timing.stop[g_timing.used++], s);
    if (e != hipSuccess) return device_fail(e, "timing event");
  }
  if (!fused) {  // the fused calls combine pieces and partials in one pass instead
    e = dcp::launch_finish_units(a, s);
    if (e != hipSuccess) return device_fail(e, "finish launch");
  }
  *plan_out = plan;
  *args_out = a;
  return DCP_OK;
}

}  // namespace

extern "C" {

int32_t dcp_abi_version(void) { return DCP_ABI_VERSION; }

const char* dcp_status_string(dcp_status s) {
  switch (s) {
    case DCP_OK: return "ok";
    case DCP_ERR_NULL: return "a required pointer is NULL";
    case DCP_ERR_SHAPE: return "sizes out of range or inconsistent";
    case DCP_ERR_UNSUPPORTED: return "no kernel implements this shape";
    case DCP_ERR_WORKSPACE: return "workspace too small";
    case DCP_ERR_BAD_PLAN: return "invalid sequence lengths";
    case DCP_ERR_ALIGN: return "device pointer not 16-byte aligned";
    case DCP_ERR_DEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dcp_last_error(void) { return g_last_error.c_str(); }

dcp_status dcp_plan_shards(const int32_t* seq_lens, int32_t batch, int32_t num_shards,
                           int32_t block_size, int32_t* bounds) {
  if (!seq_lens || !bounds) return fail(DCP_ERR_NULL, "seq_lens and bounds must be non-NULL");
  if (batch < 1 || num_shards < 1 || block_size < 1)
    return fail(DCP_ERR_SHAPE, "batch (%d), num_shards (%d) and block_size (%d) must be >= 1",
                batch, num_shards, block_size);
  for (int32_t b = 0; b < batch; ++b)
    if (seq_lens[b] < 0) return fail(DCP_ERR_BAD_PLAN, "seq_lens[%d] = %d is negative", b, seq_lens[b]);
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    const int64_t pages = (L + block_size - 1) / block_size;
    const int64_t per = (pages + num_shards - 1) / num_shards;
    for (int32_t s = 0; s < num_shards; ++s) {
      const int64_t a = (int64_t)s * per * block_size, e = (int64_t)(s + 1) * per * block_size;
      bounds[2 * ((int64_t)b * num_shards + s)] = (int32_t)(a < L ? a : L);
      bounds[2 * ((int64_t)b * num_shards + s) + 1] = (int32_t)(e < L ? e : L);
    }
  }
  return ok();
}

dcp_status dcp_plan_shards_device(const int32_t* seq_lens, int32_t batch, int32_t num_shards,
                                  int32_t block_size, int32_t* bounds, void* stream) {
  if (!seq_lens || !bounds) return fail(DCP_ERR_NULL, "seq_lens and bounds must be non-NULL");
  if (batch < 1 || num_shards < 1 || block_size < 1)
    return fail(DCP_ERR_SHAPE, "batch (%d), num_shards (%d) and block_size (%d) must be >= 1",
                batch, num_shards, block_size);
  hipError_t e = dcp::launch_plan_device(seq_lens, batch, num_shards, block_size, bounds,
                                         as_stream(stream));
  if (e != hipSuccess) return device_fail(e, "plan launch");
  return ok();
}

dcp_status dcp_workspace_bytes_multi(const dcp_attn_shape* shape, int32_t q_len, size_t* bytes) {
  if (!bytes) return fail(DCP_ERR_NULL, "bytes is NULL");
  dcp::Plan plan;
  dcp_status st = make_plan(shape, q_len, &plan);
  if (st != DCP_OK) return st;
  size_t total = plan.ws.total;
  // a call that runs in two passes reuses the workspace for each
  const int32_t ta = split_tokens(shape, q_len);
  if (ta > 0) {
    for (const int32_t t : {ta, q_len - ta}) {
      dcp::Plan p2;
      st = make_plan(shape, t, &p2);
      if (st != DCP_OK) return st;
      if (p2.ws.total > total) total = p2.ws.total;
    }
  }
  *bytes = total;
  return ok();
}

dcp_status dcp_workspace_bytes(const dcp_attn_shape* shape, size_t* bytes) {
  return dcp_workspace_bytes_multi(shape, 1, bytes);
}

dcp_status dcp_decode_attn_multi_partial(const dcp_attn_shape* shape, int32_t q_len,
                                         const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_table, const int32_t* bounds,
                                         float* part_o, float* part_lse, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  {
    dcp::Plan p0;  // the shape and q_len checks, before the pass split reads them
    const dcp_status st = make_plan(shape, q_len, &p0);
    if (st != DCP_OK) return st;
  }
  // one pass, or two (see split_tokens), each writing its own rows of part_o and part_lse
  const int32_t ta = split_tokens(shape, q_len);
  const int32_t passes = ta > 0 ? 2 : 1;
  for (int32_t i = 0; i < passes; ++i) {
    const int32_t j0 = i == 0 ? 0 : ta;
    const int32_t t = passes == 1 ? q_len : (i == 0 ? ta : q_len - ta);
    dcp::Plan plan;
    dcp::AttnArgs a;
    const dcp_status st = run_partials(shape, t, q, k_cache, v_cache, block_table, bounds, part_o,
                                       part_lse, workspace, workspace_bytes, stream, &plan, &a,
                                       false, j0, q_len);
    if (st != DCP_OK) return st;
  }
  return ok();
}

dcp_status dcp_decode_attn_partial(const dcp_attn_shape* shape, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* bounds,
                                   float* part_o, float* part_lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return dcp_decode_attn_multi_partial(shape, 1, q, k_cache, v_cache, block_table, bounds,
                                       part_o, part_lse, workspace, workspace_bytes, stream);
}

dcp_status dcp_merge_lse(int32_t batch, int32_t num_shards, int32_t num_heads, int32_t head_dim_v,
                         const float* part_o, const float* part_lse, float* out, float* out_lse,
                         void* stream) {
  if (!part_o || !part_lse || !out)
    return fail(DCP_ERR_NULL, "part_o, part_lse and out must be non-NULL");
  if (batch < 1 || num_shards < 1 || num_heads < 1 || head_dim_v < 1 || head_dim_v % 4 != 0)
    return fail(DCP_ERR_SHAPE, "batch, num_shards, num_heads >= 1 and head_dim_v a positive "
                "multiple of 4 required");
  if (!aligned16(part_o) || !aligned16(out))
    return fail(DCP_ERR_ALIGN, "part_o and out must be 16-byte aligned");
  hipError_t e = dcp::launch_merge(batch, num_shards, num_heads, head_dim_v, part_o, part_lse,
                                   out, out_lse, as_stream(stream));
  if (e != hipSuccess) return device_fail(e, "merge launch");
  return ok();
}

dcp_status dcp_decode_attn_multi(const dcp_attn_shape* shape, int32_t q_len, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* bounds,
                                 void* workspace, size_t workspace_bytes, float* out,
                                 float* out_lse, void* stream) {
  if (!out) return fail(DCP_ERR_NULL, "out must be non-NULL");
  if (!aligned16(out)) return fail(DCP_ERR_ALIGN, "out must be 16-byte aligned");
  {
    dcp::Plan p0;  // the shape and q_len checks, before the pass split reads them
    const dcp_status st = make_plan(shape, q_len, &p0);
    if (st != DCP_OK) return st;
  }
  // one pass, or two (see split_tokens) run one after the other on the stream, each writing
  // its own rows of out and out_lse; the second reuses the workspace after the first's combine
  const int32_t ta = split_tokens(shape, q_len);
  const int32_t passes = ta > 0 ? 2 : 1;
  for (int32_t i = 0; i < passes; ++i) {
    const int32_t j0 = i == 0 ? 0 : ta;
    const int32_t t = passes == 1 ? q_len : (i == 0 ? ta : q_len - ta);
    dcp::Plan plan;
    dcp::AttnArgs a;
    dcp_status st = run_partials(shape, t, q, k_cache, v_cache, block_table, bounds, nullptr,
                                 nullptr, workspace, workspace_bytes, stream, &plan, &a, true,
                                 j0, q_len);
    if (st != DCP_OK) return st;
    hipError_t e = dcp::launch_combine(a, out, out_lse, as_stream(stream));
    if (e != hipSuccess) return device_fail(e, "combine launch");
  }
  return ok();
}

dcp_status dcp_decode_attn(const dcp_attn_shape* shape, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* block_table, const int32_t* bounds,
                           void* workspace, size_t workspace_bytes, float* out, float* out_lse,
                           void* stream) {
  return dcp_decode_attn_multi(shape, 1, q, k_cache, v_cache, block_table, bounds, workspace,
                               workspace_bytes, out, out_lse, stream);
}

dcp_status dcp_decode_attn_noalloc(const dcp_attn_shape* shape, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* bounds, float* out,
                                   float* out_lse, void* stream) {
  dcp::Plan plan;
  dcp_status st = make_plan(shape, 1, &plan);
  if (st != DCP_OK) return st;
  if (!q || !k_cache || !block_table || !bounds || !out)
    return fail(DCP_ERR_NULL, "q, k_cache, block_table, bounds and out must be non-NULL");
  if (plan.ws.total > DCP_NOALLOC_SCRATCH_BYTES)
    return fail(DCP_ERR_WORKSPACE,
                "this shape needs %zu bytes of workspace; the static scratch of "
                "dcp_decode_attn_noalloc holds %zu (use dcp_decode_attn with a workspace)",
                plan.ws.total, (size_t)DCP_NOALLOC_SCRATCH_BYTES);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(DCP_ERR_DEVICE, "device %d: the static scratch is tracked for devices 0..%d",
                dev, kMaxScratchDevices - 1);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      // first call on this device (the current one): its copy of the array
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return device_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p) return fail(DCP_ERR_DEVICE, "hipGetSymbolAddress(scratch) returned NULL");
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  // every word the kernels read is written earlier in the same call (the schedule kernel
  // clears the flags, the zero row and the recomputation marks), so nothing is cleared here
  return dcp_decode_attn(shape, q, k_cache, v_cache, block_table, bounds, ws,
                         DCP_NOALLOC_SCRATCH_BYTES, out, out_lse, stream);
}

dcp_status dcp_read_device_flags(const void* workspace, int32_t* flags, void* stream) {
  if (!workspace || !flags) return fail(DCP_ERR_NULL, "workspace and flags must be non-NULL");
  hipError_t e = hipMemcpyAsync(flags, workspace, sizeof(int32_t), hipMemcpyDeviceToHost,
                                as_stream(stream));
  if (e == hipSuccess) e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return device_fail(e, "flag read");
  return ok();
}

dcp_status dcp_debug_gather_shard(const dcp_attn_shape* shape, const void* cache,
                                  const int32_t* block_table, const int32_t* bounds, int32_t b,
                                  int32_t s, int32_t kv_head, void* dst, int32_t max_rows,
                                  void* stream) {
  dcp_status st = check_shape(shape);
  if (st != DCP_OK) return st;
  if (!cache || !block_table || !bounds || !dst)
    return fail(DCP_ERR_NULL, "cache, block_table, bounds and dst must be non-NULL");
  if (b < 0 || b >= shape->batch || s < 0 || s >= shape->num_shards || kv_head < 0 ||
      kv_head >= shape->num_kv_heads || max_rows < 0)
    return fail(DCP_ERR_SHAPE, "b, s or kv_head out of range, or max_rows < 0");
  hipError_t e = dcp::launch_debug_gather(*shape, cache, block_table, bounds, b, s, kv_head, dst,
                                          max_rows, as_stream(stream));
  if (e != hipSuccess) return device_fail(e, "gather launch");
  return ok();
}

dcp_status dcp_append_kv(const dcp_attn_shape* shape, const int32_t* seq_lens,
                         const void* new_k, const void* new_v, const int32_t* block_table,
                         void* k_cache, void* v_cache, int32_t* owner, void* stream) {
  dcp_status st = check_shape(shape);
  if (st != DCP_OK) return st;
  if (!seq_lens || !new_k || !block_table || !k_cache)
    return fail(DCP_ERR_NULL, "seq_lens, new_k, block_table and k_cache must be non-NULL");
  const bool gqa = shape->kv_kind == DCP_KV_GQA;
  if (gqa && (!new_v || !v_cache)) return fail(DCP_ERR_NULL, "GQA needs new_v and v_cache");
  if (!gqa && (new_v || v_cache))
    return fail(DCP_ERR_SHAPE, "MLA stores one latent row; new_v and v_cache must be NULL");
  if (!aligned16(new_k) || !aligned16(k_cache) || (gqa && (!aligned16(new_v) || !aligned16(v_cache))))
    return fail(DCP_ERR_ALIGN, "new rows and caches must be 16-byte aligned");
  const int32_t esize = shape->dtype == DCP_F32 ? 4 : 2;
  if ((shape->head_dim_qk * esize) % 16 != 0 || (gqa && (shape->head_dim_v * esize) % 16 != 0))
    return fail(DCP_ERR_UNSUPPORTED, "cache rows must be whole 16-byte chunks (head_dim %d/%d)",
                shape->head_dim_qk, shape->head_dim_v);
  hipError_t e = dcp::launch_append_kv(*shape, seq_lens, new_k, new_v, block_table, k_cache,
                                       v_cache, owner, as_stream(stream));
  if (e != hipSuccess) return device_fail(e, "append launch");
  return ok();
}

dcp_status dcp_hbm_read_ceiling(const void* src, size_t bytes, int32_t* sink, void* stream) {
  if (!src || !sink) return fail(DCP_ERR_NULL, "src and sink must be non-NULL");
  if (!aligned16(src)) return fail(DCP_ERR_ALIGN, "src must be 16-byte aligned");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(DCP_ERR_SHAPE, "bytes (%zu) must be a positive multiple of 16", bytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_fail(e, "hipGetDevice");
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return device_fail(e, "hipDeviceGetAttribute");
  // two workgroups of 8 waves per CU
  e = dcp::launch_stream_read(src, bytes, sink, 2 * (cus > 0 ? cus : 256), as_stream(stream));
  if (e != hipSuccess) return device_fail(e, "stream-read launch");
  return ok();
}

dcp_status dcp_kernel_timing_begin(int32_t max_launches) {
  if (max_launches < 1) return fail(DCP_ERR_SHAPE, "max_launches must be >= 1");
  destroy_timing_events();
  for (int32_t i = 0; i < max_launches; ++i) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) {
      if (a) (void)hipEventDestroy(a);
      destroy_timing_events();
      return device_fail(e, "hipEventCreate");
    }
    g_timing.start.push_back(a);
    g_timing.stop.push_back(b);
  }
  g_timing.on = true;
  return ok();
}

dcp_status dcp_kernel_timing_end(int32_t* launches, float* total_ms) {
  if (!launches || !total_ms) return fail(DCP_ERR_NULL, "launches and total_ms must be non-NULL");
  float sum = 0.f;
  for (size_t i = 0; i < g_timing.used; ++i) {
    hipError_t e = hipEventSynchronize(g_timing.stop[i]);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_timing.start[i], g_timing.stop[i]);
    if (e != hipSuccess) {
      destroy_timing_events();
      return device_fail(e, "timing readback");
    }
    sum += ms;
  }
  *launches = (int32_t)g_timing.used;
  *total_ms = sum;
  destroy_timing_events();
  return ok();
}

}  // extern "C"
