"""CPU float64 oracle for sequence-sharded paged decode attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the product path never
calls it and shares no code with it.

What it computes, and where each step comes from:

* Shard plan (``plan_shards``). The Qiita page (section "トークンの区間でGPU
  に割り振る") places each request's KV on the DCP ranks by token position:
  every rank owns one contiguous range, e.g. a 200K-token request on 4 GPUs
  gives 0-50K, 50K-100K and so on. The naphjohn blog (section 2, "Core
  mechanism") writes the same range as [start:end]. The pages do not say where
  the cuts fall for lengths that do not divide; the reading taken here cuts at
  whole KV pages: P = ceil(L / bs) pages, ceil(P / S) pages per shard, the last
  shard ragged and trailing shards possibly empty. Ranges are half-open.
* Paged KV (``gather_*``). vLLM keeps the cache in non-contiguous blocks (news
  summary page, paragraph on PagedAttention); token t of sequence b lives in
  physical page block_table[b, t // bs] at slot t % bs.
* Partial attention (``attention`` on a shard's rows). The Qiita page's
  three-step description has each rank attend with the 1-token decode query
  over only its local KV slice, producing a partial result; the blog's
  section 2 says the same. The partial result is taken to be the softmax
  output over the slice together with its log-sum-exp of the scaled scores
  (natural log).
* Several query tokens per request (``partial_attention_multi``). Both pages
  list speculative decoding / MTP as work that DCP is to be combined with
  (Qiita, section "実務でどう見るか"; naphjohn blog, section 5). Such a step
  scores q_len new tokens at once. The reading taken here: they are the
  request's q_len newest positions L - q_len .. L - 1 (L = the end of the
  ranges that cover the request), their KV is already in the cache, and token
  j attends to every position up to and including its own (causal order).
  Each shard's partial is then the softmax over the shard's tokens that the
  row may see, and the same LSE merge gives the causal attention result. The
  blog's section 4 also has DCP reach chunked and cached prefill: a chunk of
  new tokens scored against the sharded cache is the same computation with a
  larger q_len.
* KV append (``append_token``). Decode makes one token per step and each
  rank keeps only its own slice of the KV (naphjohn blog, section 4, the
  decode bullet; Qiita token-range section). The new token of a request that
  already holds L tokens has position L, so under the paged layout it is
  stored at slot L % bs of page block_table[b, L // bs]; the shard that owns
  it is the one whose range in the plan of the grown length L + 1 contains L
  (always the last non-empty shard). Positions with no block-table entry or
  entries outside the page pool are reported, not written.
* Merge (``merge_lse``). The partial results are combined with online-softmax
  re-weighting and must give the full attention result (Qiita three-step
  paragraph; blog section 2). The re-weighting written out is the LSE merge:
  M = max_s LSE_s, LSE = M + ln sum_s exp(LSE_s - M),
  O = sum_s exp(LSE_s - LSE) O_s; shards with LSE = -inf contribute nothing,
  and if every shard is empty O = 0 and LSE = -inf.

Inputs are upcast exactly (bf16 bit patterns and float32 values both convert
to float64 without rounding), so input quantisation is never charged to the
GPU path. GQA query head h reads KV head h // G (contiguous groups). For MLA
the value of token t is the first ``head_dim_v`` dims of its cached latent row.
"""

from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- conversions

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16/int16) as float64."""
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of stored values; dtype is "bf16" (bit patterns) or "f32"."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- shard plan

def plan_shards(seq_lens, num_shards: int, block_size: int) -> np.ndarray:
    """Page-aligned contiguous shard ranges, int64 [B, S, 2] of (start, end).

    Shard s of a length-L request covers tokens [min(L, s*k*bs), min(L, (s+1)*k*bs))
    with k = ceil(ceil(L/bs) / S) pages per shard.
    """
    if num_shards < 1 or block_size < 1:
        raise ValueError("num_shards and block_size must be >= 1")
    out = np.zeros((len(seq_lens), num_shards, 2), dtype=np.int64)
    for b, L in enumerate(seq_lens):
        L = int(L)
        if L < 0:
            raise ValueError("negative length")
        pages = -(-L // block_size)
        per_shard = -(-pages // num_shards)
        for s in range(num_shards):
            out[b, s, 0] = min(L, s * per_shard * block_size)
            out[b, s, 1] = min(L, (s + 1) * per_shard * block_size)
    return out


# ---------------------------------------------------------------- paged gather

def gather_gqa(cache: np.ndarray, block_table: np.ndarray, b: int, kv_head: int,
               start: int, end: int, block_size: int) -> np.ndarray:
    """Rows of tokens [start, end) of sequence b, KV head kv_head, from a
    [num_blocks, Hkv, bs, D] cache (stored values, not converted)."""
    rows = [cache[block_table[b, t // block_size], kv_head, t % block_size]
            for t in range(start, end)]
    if not rows:
        return cache[:0, 0, 0]
    return np.stack(rows)


def gather_mla(cache: np.ndarray, block_table: np.ndarray, b: int, start: int, end: int,
               block_size: int) -> np.ndarray:
    """Rows of tokens [start, end) of sequence b from a [num_blocks, bs, Dqk] cache."""
    rows = [cache[block_table[b, t // block_size], t % block_size] for t in range(start, end)]
    if not rows:
        return cache[:0, 0]
    return np.stack(rows)


def _gather_fast(cache, block_table, b, start, end, bs, kv_head=None):
    """Same rows as gather_gqa/gather_mla, by whole pages (for large inputs)."""
    if end <= start:
        return gather_mla(cache, block_table, b, 0, 0, bs) if kv_head is None else \
            gather_gqa(cache, block_table, b, kv_head, 0, 0, bs)
    p0, p1 = start // bs, -(-end // bs)
    pages = block_table[b, p0:p1]
    blk = cache[pages] if kv_head is None else cache[pages, kv_head]
    rows = blk.reshape((-1,) + blk.shape[2:])
    off = start - p0 * bs
    return rows[off:off + (end - start)]


# ---------------------------------------------------------------- attention

def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Softmax attention of H query rows over n key/value rows, float64.

    s_ht = scale * <q_h, k_t>;  LSE_h = ln sum_t exp(s_ht);  O_h = sum_t exp(s_ht - LSE_h) v_t.
    With n = 0: O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    H = q.shape[0]
    dv = v.shape[1]
    if k.shape[0] == 0:
        return np.zeros((H, dv)), np.full(H, -np.inf)
    s = scale * (q @ np.asarray(k, dtype=np.float64).T)
    m = s.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    o = np.exp(s - lse[:, None]) @ np.asarray(v, dtype=np.float64)
    return o, lse


def merge_lse(part_o: np.ndarray, part_lse: np.ndarray):
    """LSE merge over the shard axis.

    part_o [..., S, H, Dv], part_lse [..., S, H] -> (O [..., H, Dv], LSE [..., H]).
    """
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    M = part_lse.max(axis=-2)                       # [..., H]
    empty = np.isneginf(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.exp(part_lse - Msafe[..., None, :])      # exp(-inf) = 0 for empty shards
    total = w.sum(axis=-2)
    lse = np.where(empty, -np.inf, Msafe + np.log(np.where(empty, 1.0, total)))
    lse_safe = np.where(empty, 0.0, lse)
    wt = np.exp(part_lse - lse_safe[..., None, :])  # exp(LSE_s - LSE)
    wt = np.where(empty[..., None, :], 0.0, wt)
    o = (wt[..., None] * part_o).sum(axis=-3)
    return o, lse


# ---------------------------------------------------------------- whole path

def _q_rows(q, b, h0, h1, dtype):
    return as_f64(q[b, h0:h1], dtype)


def partial_attention(kind: str, dtype: str, q, caches, block_table, bounds, block_size: int,
                      scale: float, head_dim_v: int, seqs=None):
    """Per-shard partials (O_s, LSE_s) for every (b, s) (or the listed seqs).

    kind "gqa": caches = (k_cache [N, Hkv, bs, D], v_cache same).
    kind "mla": caches = (kv_cache [N, bs, Dqk],); V = first head_dim_v dims.
    Returns part_o [B, S, Hq, Dv] and part_lse [B, S, Hq] (rows of sequences
    not in `seqs` stay NaN).
    """
    B, Hq = q.shape[0], q.shape[1]
    S = bounds.shape[1]
    part_o = np.full((B, S, Hq, head_dim_v), np.nan)
    part_lse = np.full((B, S, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        for s in range(S):
            start, end = int(bounds[b, s, 0]), int(bounds[b, s, 1])
            if kind == "mla":
                rows = as_f64(_gather_fast(caches[0], block_table, b, start, end, block_size), dtype)
                o, lse = attention(_q_rows(q, b, 0, Hq, dtype), rows, rows[:, :head_dim_v], scale)
                part_o[b, s], part_lse[b, s] = o, lse
            else:
                k_cache, v_cache = caches
                Hkv = k_cache.shape[1]
                G = Hq // Hkv
                for g in range(Hkv):
                    k = as_f64(_gather_fast(k_cache, block_table, b, start, end, block_size, g), dtype)
                    v = as_f64(_gather_fast(v_cache, block_table, b, start, end, block_size, g), dtype)
                    o, lse = attention(_q_rows(q, b, g * G, (g + 1) * G, dtype), k, v, scale)
                    part_o[b, s, g * G:(g + 1) * G] = o
                    part_lse[b, s, g * G:(g + 1) * G] = lse
    return part_o, part_lse


def full_attention(kind: str, dtype: str, q, caches, block_table, seq_lens, block_size: int,
                   scale: float, head_dim_v: int, seqs=None):
    """Unsharded attention over tokens [0, L_b): O [B, Hq, Dv], LSE [B, Hq]."""
    bounds = np.zeros((len(seq_lens), 1, 2), dtype=np.int64)
    bounds[:, 0, 1] = np.asarray(seq_lens, dtype=np.int64)
    o, lse = partial_attention(kind, dtype, q, caches, block_table, bounds, block_size, scale,
                               head_dim_v, seqs)
    return o[:, 0], lse[:, 0]


def sharded_attention(kind, dtype, q, caches, block_table, seq_lens, num_shards, block_size,
                      scale, head_dim_v, seqs=None):
    """Plan, per-shard partials, merge: returns (bounds, part_o, part_lse, O, LSE)."""
    bounds = plan_shards(seq_lens, num_shards, block_size)
    part_o, part_lse = partial_attention(kind, dtype, q, caches, block_table, bounds, block_size,
                                         scale, head_dim_v, seqs)
    o, lse = merge_lse(part_o, part_lse)
    return bounds, part_o, part_lse, o, lse


# ---------------------------------------------------------------- several query tokens

def partial_attention_multi(kind: str, dtype: str, q, caches, block_table, bounds,
                            block_size: int, scale: float, head_dim_v: int, seqs=None,
                            tokens=None):
    """Per-shard partials for q_len query tokens per request, with causal visibility.

    q [B, q_len, Hq, Dqk]; bounds [B, S, 2]. With L_b the largest end among request b's
    ranges, query token j sits at position L_b - q_len + j and sees token t only when
    t <= L_b - q_len + j. Returns part_o [B, S, q_len, Hq, Dv] and part_lse [B, S, q_len, Hq]
    (a row that sees nothing in a shard gets O = 0, LSE = -inf; rows of sequences not in
    `seqs`, and query tokens j not in `tokens` when it is given, stay NaN).
    """
    B, q_len, Hq = q.shape[0], q.shape[1], q.shape[2]
    S = bounds.shape[1]
    part_o = np.full((B, S, q_len, Hq, head_dim_v), np.nan)
    part_lse = np.full((B, S, q_len, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(np.max(bounds[b, :, 1])) if S else 0
        for s in range(S):
            start, end = int(bounds[b, s, 0]), int(bounds[b, s, 1])
            for j in (range(q_len) if tokens is None else tokens):
                last = min(end, L - q_len + j + 1)   # exclusive end of the visible part
                stop = max(start, last)
                if kind == "mla":
                    rows = as_f64(_gather_fast(caches[0], block_table, b, start, stop,
                                               block_size), dtype)
                    o, lse = attention(as_f64(q[b, j], dtype), rows, rows[:, :head_dim_v], scale)
                    part_o[b, s, j], part_lse[b, s, j] = o, lse
                else:
                    k_cache, v_cache = caches
                    G = Hq // k_cache.shape[1]
                    for g in range(k_cache.shape[1]):
                        k = as_f64(_gather_fast(k_cache, block_table, b, start, stop,
                                                block_size, g), dtype)
                        v = as_f64(_gather_fast(v_cache, block_table, b, start, stop,
                                                block_size, g), dtype)
                        o, lse = attention(as_f64(q[b, j, g * G:(g + 1) * G], dtype), k, v, scale)
                        part_o[b, s, j, g * G:(g + 1) * G] = o
                        part_lse[b, s, j, g * G:(g + 1) * G] = lse
    return part_o, part_lse


def sharded_attention_multi(kind, dtype, q, caches, block_table, seq_lens, num_shards,
                            block_size, scale, head_dim_v, seqs=None):
    """Plan of seq_lens, causal partials, merge: (bounds, part_o, part_lse, O, LSE) with
    O [B, q_len, Hq, Dv] and LSE [B, q_len, Hq]."""
    bounds = plan_shards(seq_lens, num_shards, block_size)
    part_o, part_lse = partial_attention_multi(kind, dtype, q, caches, block_table, bounds,
                                               block_size, scale, head_dim_v, seqs)
    B, S, T, H, Dv = part_o.shape
    o, lse = merge_lse(part_o.reshape(B, S, T * H, Dv), part_lse.reshape(B, S, T * H))
    return bounds, part_o, part_lse, o.reshape(B, T, H, Dv), lse.reshape(B, T, H)

# ---------------------------------------------------------------- KV append

def append_token(kind: str, caches, new_rows, block_table, seq_lens, block_size: int,
                 num_shards: int):
    """Store each request's newly decoded token in its page and name the owning shard.

    kind "gqa": caches = (k_cache [N, Hkv, bs, D], v_cache [N, Hkv, bs, Dv]) and
    new_rows = (new_k [B, Hkv, D], new_v [B, Hkv, Dv]); kind "mla": caches = (latent
    [N, bs, D],) and new_rows = (new_latent [B, D],). seq_lens[b] = L_b tokens already
    cached; the new token takes position L_b.

    Returns (copies of the caches with the rows stored, owner int64 [B]): owner[b] is the
    shard holding position L_b in plan_shards of L_b + 1 tokens; -1 when L_b < 0 or
    L_b // bs is past the block table's row, -2 when the table entry is not a page in
    [0, N). Nothing is stored for a request whose owner is negative. Requests are stored
    in order of b, so if two of them name the same (page, slot) the later one stays.
    """
    out = tuple(np.array(c, copy=True) for c in caches)
    table = np.asarray(block_table)
    max_blocks = table.shape[1]
    n_pages = out[0].shape[0]
    owner = np.zeros(len(seq_lens), dtype=np.int64)
    for b, L in enumerate(seq_lens):
        L = int(L)
        if L < 0 or L // block_size >= max_blocks:
            owner[b] = -1
            continue
        page = int(table[b, L // block_size])
        if page < 0 or page >= n_pages:
            owner[b] = -2
            continue
        slot = L % block_size
        ranges = plan_shards([L + 1], num_shards, block_size)[0]
        owner[b] = next(s for s in range(num_shards) if ranges[s, 0] <= L < ranges[s, 1])
        if kind == "mla":
            out[0][page, slot] = new_rows[0][b]
        else:
            for i in range(2):
                out[i][page, :, slot] = new_rows[i][b]
    return out, owner
