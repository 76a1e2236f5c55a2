"""Plant plausible mistakes in the oracle (on the CPU) and require that at
least one pin fails for each; a pin set that lets a mistake through is too
weak to trust the oracle by."""

import math

import numpy as np
import pytest

import oracle_pins as P
from oracle import oracle as O

_attn = O.attention
_merge = O.merge_lse
_plan = O.plan_shards
_gq = O.gather_gqa
_gm = O.gather_mla
_gf = O._gather_fast
_partial = O.partial_attention
_up = O.bf16_bits_to_f64
_append = O.append_token
_multi = O.partial_attention_multi


def m_attn_no_scale(q, k, v, scale):
    return _attn(q, k, v, 1.0)


def m_attn_log2(q, k, v, scale):
    o, lse = _attn(q, k, v, scale)
    return o, lse / math.log(2.0)


def m_attn_lse_no_max(q, k, v, scale):
    o, lse = _attn(q, k, v, scale)
    if k.shape[0] == 0:
        return o, lse
    s = scale * (np.asarray(q, float) @ np.asarray(k, float).T)
    return o, lse - s.max(axis=1)


def m_attn_keys_as_values(q, k, v, scale):
    o, lse = _attn(q, k, np.asarray(k)[:, :v.shape[1]] if k.shape[1] >= v.shape[1] else v, scale)
    return o, lse


def m_attn_drop_last_token(q, k, v, scale):
    n = k.shape[0]
    return _attn(q, k[:max(0, n - 1)] if n > 1 else k, v[:max(0, n - 1)] if n > 1 else v, scale)


def m_merge_unnormalised(po, pl):
    po, pl = np.asarray(po, float), np.asarray(pl, float)
    M = pl.max(axis=-2)
    w = np.exp(pl - np.where(np.isneginf(M), 0, M)[..., None, :])
    return (w[..., None] * po).sum(axis=-3), M


def m_merge_sign(po, pl):
    return _merge(po, -np.asarray(pl, float))


def m_merge_plain_mean(po, pl):
    o, lse = _merge(po, pl)
    return np.asarray(po, float).mean(axis=-3), lse


def m_merge_no_empty_guard(po, pl):
    po, pl = np.asarray(po, float), np.asarray(pl, float)
    M = pl.max(axis=-2)
    lse = M + np.log(np.exp(pl - M[..., None, :]).sum(axis=-2))
    w = np.exp(pl - lse[..., None, :])
    return (w[..., None] * po).sum(axis=-3), lse


def m_plan_floor(seq_lens, S, bs):
    out = np.zeros((len(seq_lens), S, 2), dtype=np.int64)
    for b, L in enumerate(seq_lens):
        pages = -(-int(L) // bs)
        k = max(1, pages // S)
        for s in range(S):
            out[b, s] = (min(L, s * k * bs), min(L, (s + 1) * k * bs))
    return out


def m_plan_token_split(seq_lens, S, bs):
    out = np.zeros((len(seq_lens), S, 2), dtype=np.int64)
    for b, L in enumerate(seq_lens):
        k = -(-int(L) // S)
        for s in range(S):
            out[b, s] = (min(L, s * k), min(L, (s + 1) * k))
    return out


def m_plan_no_clamp(seq_lens, S, bs):
    out = _plan(seq_lens, S, bs)
    for b, L in enumerate(seq_lens):
        pages = -(-int(L) // bs)
        k = -(-pages // S)
        out[b, S - 1, 1] = S * k * bs if L else 0
    return out


def m_gather_gqa_swapped(cache, table, b, g, a, e, bs):
    rows = [cache[table[b, t % bs], g, t // bs] for t in range(a, e)]
    return np.stack(rows) if rows else cache[:0, 0, 0]


def m_gather_mla_off_by_one(cache, table, b, a, e, bs):
    return _gm(cache, table, b, a + 1, e + 1, bs) if e > a else _gm(cache, table, b, a, e, bs)


def m_gather_fast_shift(cache, table, b, a, e, bs, kv_head=None):
    rows = _gf(cache, table, b, a, e, bs, kv_head)
    return np.roll(rows, 1, axis=0)


def m_partial_interleaved_heads(kind, dtype, q, caches, table, bounds, bs, scale, dv, seqs=None):
    if kind != "gqa":
        return _partial(kind, dtype, q, caches, table, bounds, bs, scale, dv, seqs)
    Hq, Hkv = q.shape[1], caches[0].shape[1]
    order = np.argsort([h % Hkv for h in range(Hq)], kind="stable")
    po, pl = _partial(kind, dtype, q[:, order], caches, table, bounds, bs, scale, dv, seqs)
    po2, pl2 = np.empty_like(po), np.empty_like(pl)
    po2[:, :, order], pl2[:, :, order] = po, pl
    return po2, pl2


def m_partial_value_suffix(kind, dtype, q, caches, table, bounds, bs, scale, dv, seqs=None):
    if kind != "mla":
        return _partial(kind, dtype, q, caches, table, bounds, bs, scale, dv, seqs)
    c = caches[0]
    rolled = np.concatenate([c[..., -dv:], c[..., : c.shape[-1] - dv]], axis=-1)
    # scores from the true rows, values from the last dv dims
    B, S = bounds.shape[:2]
    po = np.zeros((B, S, q.shape[1], dv)); pl = np.zeros((B, S, q.shape[1]))
    for b in range(B):
        for s in range(S):
            a, e = int(bounds[b, s, 0]), int(bounds[b, s, 1])
            rows = O.as_f64(_gf(c, table, b, a, e, bs), dtype)
            vals = O.as_f64(_gf(rolled, table, b, a, e, bs), dtype)[:, :dv]
            po[b, s], pl[b, s] = _attn(O.as_f64(q[b], dtype), rows, vals, scale)
    return po, pl


def m_upcast_shift15(bits):
    u = np.asarray(bits).view(np.uint16).astype(np.uint32) << 15
    return u.view(np.float32).astype(np.float64)


def m_append_slot_page_swapped(kind, caches, new_rows, table, seq_lens, bs, S):
    out = tuple(np.array(c, copy=True) for c in caches)
    _, owner = _append(kind, caches, new_rows, table, seq_lens, bs, S)
    for b, L in enumerate(seq_lens):
        if owner[b] < 0:
            continue
        page, slot = int(table[b, L % bs % table.shape[1]]), min(L // bs, bs - 1)
        if kind == "mla":
            out[0][page, slot] = new_rows[0][b]
        else:
            out[0][page, :, slot], out[1][page, :, slot] = new_rows[0][b], new_rows[1][b]
    return out, owner


def m_append_next_position(kind, caches, new_rows, table, seq_lens, bs, S):
    return _append(kind, caches, new_rows, table, [int(L) + 1 for L in seq_lens], bs, S)


def m_append_owner_from_old_length(kind, caches, new_rows, table, seq_lens, bs, S):
    out, owner = _append(kind, caches, new_rows, table, seq_lens, bs, S)
    for b, L in enumerate(seq_lens):
        if owner[b] >= 0:
            k = -(-(-(-int(L) // bs)) // S)
            owner[b] = 0 if k == 0 else min(S - 1, int(L) // (k * bs))
    return out, owner


def m_append_owner_last_shard(kind, caches, new_rows, table, seq_lens, bs, S):
    out, owner = _append(kind, caches, new_rows, table, seq_lens, bs, S)
    return out, np.where(owner >= 0, S - 1, owner)


def m_append_no_page_check(kind, caches, new_rows, table, seq_lens, bs, S):
    n = caches[0].shape[0]
    wrapped = np.where((np.asarray(table) < 0) | (np.asarray(table) >= n), 0, table)
    return _append(kind, caches, new_rows, wrapped, seq_lens, bs, S)


def m_append_k_gets_v(kind, caches, new_rows, table, seq_lens, bs, S):
    if kind != "gqa" or new_rows[0].shape != new_rows[1].shape:
        return _append(kind, caches, new_rows, table, seq_lens, bs, S)
    return _append(kind, caches, (new_rows[1], new_rows[0]), table, seq_lens, bs, S)


def _multi_with_positions(pos_of, kind, dtype, q, caches, table, bounds, bs, scale, dv,
                          seqs=None):
    """The oracle's causal partials with query token j placed at pos_of(L, T, j)."""
    B, T, Hq = q.shape[:3]
    S = bounds.shape[1]
    po = np.zeros((B, S, T, Hq, dv))
    pl = np.full((B, S, T, Hq), -np.inf)
    for b in range(B):
        L = int(np.max(bounds[b, :, 1]))
        for j in range(T):
            pos = pos_of(L, T, j)
            nb = np.array(bounds[b:b + 1], copy=True)
            nb[..., 1] = np.minimum(nb[..., 1], max(0, pos + 1))
            nb[..., 0] = np.minimum(nb[..., 0], nb[..., 1])
            o, l = _multi(kind, dtype, q[b:b + 1, j:j + 1], caches, table[b:b + 1], nb, bs, scale,
                          dv)
            po[b, :, j], pl[b, :, j] = o[0, :, 0], l[0, :, 0]
    return po, pl


def m_multi_excludes_own_token(*args, **kw):
    return _multi_with_positions(lambda L, T, j: L - T + j - 1, *args, **kw)


def m_multi_positions_from_zero(*args, **kw):
    return _multi_with_positions(lambda L, T, j: j, *args, **kw)


def m_multi_no_causal_mask(*args, **kw):
    return _multi_with_positions(lambda L, T, j: L - 1, *args, **kw)


def m_multi_tokens_reversed(*args, **kw):
    return _multi_with_positions(lambda L, T, j: L - 1 - j, *args, **kw)


MUTANTS = [
    ("attention", m_attn_no_scale),
    ("attention", m_attn_log2),
    ("attention", m_attn_lse_no_max),
    ("attention", m_attn_keys_as_values),
    ("attention", m_attn_drop_last_token),
    ("merge_lse", m_merge_unnormalised),
    ("merge_lse", m_merge_sign),
    ("merge_lse", m_merge_plain_mean),
    ("merge_lse", m_merge_no_empty_guard),
    ("plan_shards", m_plan_floor),
    ("plan_shards", m_plan_token_split),
    ("plan_shards", m_plan_no_clamp),
    ("gather_gqa", m_gather_gqa_swapped),
    ("gather_mla", m_gather_mla_off_by_one),
    ("_gather_fast", m_gather_fast_shift),
    ("partial_attention", m_partial_interleaved_heads),
    ("partial_attention", m_partial_value_suffix),
    ("bf16_bits_to_f64", m_upcast_shift15),
    ("partial_attention_multi", m_multi_excludes_own_token),
    ("partial_attention_multi", m_multi_positions_from_zero),
    ("partial_attention_multi", m_multi_no_causal_mask),
    ("partial_attention_multi", m_multi_tokens_reversed),
    ("append_token", m_append_slot_page_swapped),
    ("append_token", m_append_next_position),
    ("append_token", m_append_owner_from_old_length),
    ("append_token", m_append_owner_last_shard),
    ("append_token", m_append_no_page_check),
    ("append_token", m_append_k_gets_v),
]


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant):
    monkeypatch.setattr(O, name, mutant)
    failed = []
    with np.errstate(all="ignore"):
        for check in P.ALL_CHECKS:
            try:
                check()
            except Exception as exc:  # noqa: BLE001 - any failure counts as caught
                failed.append((check.__name__, type(exc).__name__))
    assert failed, f"no pin caught the planted mistake {mutant.__name__} in {name}"
