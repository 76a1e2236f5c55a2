"""Pins for the float64 oracle: each check compares the oracle with something
that is not the oracle (the pages' worked example, brute force in pure Python,
a library routine, closed forms, invariants). Every check raises
AssertionError on failure; tests/test_oracle.py runs them, and
tests/test_oracle_mutations.py plants mistakes in the oracle and expects one
of them to fail.

The oracle is always reached through the module attribute (``O.name``) so a
planted mistake is seen by every caller.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ plan

def check_plan_golden():
    with open(os.path.join(GOLDEN, "plan_token_ranges.json")) as f:
        spec = json.load(f)
    for case in spec["cases"]:
        got = O.plan_shards(case["seq_lens"], case["num_shards"], case["block_size"])
        assert got.tolist() == case["bounds"], (case, got.tolist())


def _plan_brute(L, S, bs):
    """Smallest per-shard page budget that fits, found by search; shards filled in order."""
    pages = 0
    while pages * bs < L:
        pages += 1
    k = 0
    while k * S < pages:
        k += 1
    out, pos = [], 0
    for _ in range(S):
        take = min(k, pages - pos)
        a = min(L, pos * bs)
        pos += take
        out.append((a, min(L, pos * bs)))
    return out


def check_plan_brute(rng=None):
    rng = rng or np.random.default_rng(7)
    cases = [(0, 3, 16), (1, 8, 64), (15, 4, 16), (16, 4, 16), (17, 4, 16), (63, 8, 64),
             (1_000_000, 16, 16), (800_000, 16, 16), (500_000, 16, 16), (200_000, 16, 16)]
    cases += [(int(rng.integers(0, 5000)), int(rng.integers(1, 33)), int(rng.choice([1, 16, 64])))
              for _ in range(300)]
    for L, S, bs in cases:
        got = O.plan_shards([L], S, bs)[0].tolist()
        exp = [list(x) for x in _plan_brute(L, S, bs)]
        assert got == exp, (L, S, bs, got, exp)
        # contiguous cover of [0, L), page-aligned interior cuts
        assert got[0][0] == 0 and got[-1][1] == L
        for (a0, a1), (b0, _) in zip(got, got[1:]):
            assert a1 == b0 and a0 <= a1
            assert a1 % bs == 0 or a1 == L


# ------------------------------------------------------------------ gather

def check_gather_example():
    """bs 4, block table [2, 0, 3]: tokens 0..9 live at (page, slot) listed by hand."""
    bs, N, Hkv = 4, 4, 2
    cache = np.zeros((N, Hkv, bs, 3), dtype=np.float32)
    for p in range(N):
        for h in range(Hkv):
            for s in range(bs):
                cache[p, h, s] = (p, h, s)
    table = np.array([[2, 0, 3]], dtype=np.int32)
    want = [(2, 0), (2, 1), (2, 2), (2, 3), (0, 0), (0, 1), (0, 2), (0, 3), (3, 0), (3, 1)]
    rows = O.gather_gqa(cache, table, 0, 1, 0, 10, bs)
    assert [(int(r[0]), int(r[2])) for r in rows] == want
    assert all(int(r[1]) == 1 for r in rows)
    rows = O.gather_gqa(cache, table, 0, 0, 3, 9, bs)
    assert [(int(r[0]), int(r[2])) for r in rows] == want[3:9]
    mla = cache[:, 0]  # [N, bs, 3]
    rows = O.gather_mla(mla, table, 0, 5, 10, bs)
    assert [(int(r[0]), int(r[2])) for r in rows] == want[5:10]


def check_gather_fast_matches():
    rng = np.random.default_rng(3)
    bs, N, Hkv, D = 16, 40, 3, 5
    cache = rng.standard_normal((N, Hkv, bs, D))
    table = rng.permutation(N).reshape(2, 20).astype(np.int32)
    for _ in range(50):
        b = int(rng.integers(0, 2))
        a = int(rng.integers(0, 320))
        e = int(rng.integers(a, 321))
        g = int(rng.integers(0, Hkv))
        assert np.array_equal(O._gather_fast(cache, table, b, a, e, bs, g),
                              O.gather_gqa(cache, table, b, g, a, e, bs))
        assert np.array_equal(O._gather_fast(cache[:, g], table, b, a, e, bs),
                              O.gather_mla(cache[:, g], table, b, a, e, bs))


def check_gather_permutation_invariant():
    """Relabelling physical pages (and the table with them) changes nothing."""
    rng = np.random.default_rng(4)
    bs, N, D = 8, 12, 4
    cache = rng.standard_normal((N, bs, D))
    table = rng.permutation(N).reshape(2, 6).astype(np.int32)
    perm = rng.permutation(N)
    cache2 = np.empty_like(cache)
    cache2[perm] = cache
    table2 = perm[table].astype(np.int32)
    for b in range(2):
        assert np.array_equal(O.gather_mla(cache, table, b, 3, 45, bs),
                              O.gather_mla(cache2, table2, b, 3, 45, bs))


# ------------------------------------------------------------------ attention

def _brute_attention(q, k, v, scale):
    """Pure-Python softmax attention with math.fsum (exact-sum) reductions."""
    H, n = len(q), len(k)
    out, lses = [], []
    for h in range(H):
        s = [scale * math.fsum(q[h][d] * k[t][d] for d in range(len(q[h]))) for t in range(n)]
        m = max(s)
        tot = math.fsum(math.exp(x - m) for x in s)
        lse = m + math.log(tot)
        w = [math.exp(x - lse) for x in s]
        out.append([math.fsum(w[t] * v[t][j] for t in range(n)) for j in range(len(v[0]))])
        lses.append(lse)
    return np.array(out), np.array(lses)


def check_attention_brute():
    rng = np.random.default_rng(11)
    for n in (1, 2, 5, 12):
        for d in (1, 3, 5):
            q = rng.standard_normal((2, d))
            k = rng.standard_normal((n, d)) * 2
            v = rng.standard_normal((n, 4))
            o, lse = O.attention(q, k, v, 0.7)
            eo, el = _brute_attention(q.tolist(), k.tolist(), v.tolist(), 0.7)
            assert np.allclose(o, eo, rtol=1e-12, atol=1e-13), (n, d)
            assert np.allclose(lse, el, rtol=1e-13, atol=1e-13), (n, d)


def check_attention_library():
    """torch's scaled_dot_product_attention and logsumexp in float64 on CPU."""
    import torch
    rng = np.random.default_rng(12)
    for n, D, Dv in ((7, 16, 16), (300, 64, 64), (129, 576, 512)):
        q = rng.standard_normal((8, D))
        k = rng.standard_normal((n, D))
        v = rng.standard_normal((n, Dv))
        scale = 1.0 / math.sqrt(D)
        o, lse = O.attention(q, k, v, scale)
        tq = torch.from_numpy(q)[None, :, None, :]
        tk = torch.from_numpy(k)[None, None].expand(1, 8, n, D)
        tv = torch.from_numpy(v)[None, None].expand(1, 8, n, Dv)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)[0, :, 0]
        ref_lse = torch.logsumexp(scale * (torch.from_numpy(q) @ torch.from_numpy(k).T), dim=1)
        assert np.allclose(o, ref.numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


def check_attention_closed_forms():
    rng = np.random.default_rng(13)
    # all keys equal: uniform weights, O = mean(V), LSE = s + ln n
    q = rng.standard_normal((3, 6))
    k1 = rng.standard_normal(6)
    n = 37
    k = np.tile(k1, (n, 1))
    v = rng.standard_normal((n, 5))
    o, lse = O.attention(q, k, v, 0.4)
    s = 0.4 * (q @ k1)
    assert np.allclose(o, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, s + math.log(n), rtol=1e-13, atol=1e-13)
    # one score 1000 above the rest: O = v_j, LSE = s_j
    q = np.zeros((1, 2)); q[0, 0] = 1.0
    k = rng.standard_normal((9, 2)) * 0.1
    j = 4
    k[j, 0] = 1000.0
    v = rng.standard_normal((9, 3))
    o, lse = O.attention(q, k, v, 1.0)
    assert np.array_equal(o[0], v[j])
    assert abs(lse[0] - k[j, 0]) < 1e-9
    # empty range
    o, lse = O.attention(q, k[:0], v[:0], 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def check_attention_laws():
    rng = np.random.default_rng(14)
    q = rng.standard_normal((4, 8))
    k = rng.standard_normal((20, 8))
    v = rng.standard_normal((20, 6))
    o, lse = O.attention(q, k, v, 0.3)
    # V-affine: O(aV + b) = a O + b
    o2, lse2 = O.attention(q, k, 2.5 * v + 1.25, 0.3)
    assert np.allclose(o2, 2.5 * o + 1.25, rtol=1e-12, atol=1e-12)
    assert np.array_equal(lse, lse2)
    # the scale multiplies the scores: scale c on q == scale 1 on c*q
    o3, lse3 = O.attention(0.3 * q, k, v, 1.0)
    assert np.allclose(o3, o, rtol=1e-12, atol=1e-13) and np.allclose(lse3, lse, rtol=1e-13)
    # weights sum to one: V = all-ones gives O = 1
    o4, _ = O.attention(q, k, np.ones_like(v), 0.3)
    assert np.allclose(o4, 1.0, rtol=1e-13)


# ------------------------------------------------------------------ merge

def _random_partition(n, S, rng, allow_empty=True):
    cuts = np.sort(rng.integers(0 if allow_empty else 1, n + 1, size=S - 1))
    edges = [0] + cuts.tolist() + [n]
    return list(zip(edges[:-1], edges[1:]))


def check_merge_partition_invariance():
    rng = np.random.default_rng(15)
    for trial in range(40):
        n = int(rng.integers(1, 200))
        q = rng.standard_normal((5, 7))
        k = rng.standard_normal((n, 7)) * (3 if trial % 2 else 1)
        v = rng.standard_normal((n, 4))
        full_o, full_lse = O.attention(q, k, v, 0.5)
        kinds = [1, n, int(rng.integers(1, 40))]
        for S in kinds:
            parts = ([(t, t + 1) for t in range(n)] if S == n else _random_partition(n, S, rng))
            po = np.stack([O.attention(q, k[a:b], v[a:b], 0.5)[0] for a, b in parts])
            pl = np.stack([O.attention(q, k[a:b], v[a:b], 0.5)[1] for a, b in parts])
            mo, ml = O.merge_lse(po, pl)
            assert np.allclose(mo, full_o, rtol=1e-11, atol=1e-12), (trial, S)
            assert np.allclose(ml, full_lse, rtol=1e-12, atol=1e-12), (trial, S)


def check_merge_associative_and_edge_cases():
    rng = np.random.default_rng(16)
    po = rng.standard_normal((6, 3, 4))
    pl = rng.standard_normal((6, 3)) * 5
    pl[2] = -np.inf
    po[2] = 0.0
    o, lse = O.merge_lse(po, pl)
    oa, la = O.merge_lse(po[:3], pl[:3])
    ob, lb = O.merge_lse(po[3:], pl[3:])
    o2, l2 = O.merge_lse(np.stack([oa, ob]), np.stack([la, lb]))
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-13) and np.allclose(lse, l2, rtol=1e-13)
    # single shard: identity
    o1, l1 = O.merge_lse(po[:1], pl[:1])
    assert np.allclose(o1, po[0], rtol=1e-14, atol=0) and np.allclose(l1, pl[0], rtol=1e-14)
    # two shards with equal LSE: plain average, LSE + ln 2
    a, b = rng.standard_normal((3, 4)), rng.standard_normal((3, 4))
    lsev = rng.standard_normal(3)
    o, lse = O.merge_lse(np.stack([a, b]), np.stack([lsev, lsev]))
    assert np.allclose(o, (a + b) / 2, rtol=1e-13, atol=1e-14)
    assert np.allclose(lse, lsev + math.log(2.0), rtol=1e-13, atol=1e-14)
    # all shards empty
    o, lse = O.merge_lse(np.zeros((4, 3, 2)), np.full((4, 3), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------------------------ whole path

def check_gqa_head_groups():
    """Query head h reads KV head h // G: give KV head g all values equal to g."""
    bs, Hkv, G, D = 4, 3, 2, 4
    N = 6
    rng = np.random.default_rng(17)
    k = rng.standard_normal((N, Hkv, bs, D)).astype(np.float32)
    v = np.zeros((N, Hkv, bs, D), dtype=np.float32)
    for g in range(Hkv):
        v[:, g] = g
    q = rng.standard_normal((1, Hkv * G, D)).astype(np.float32)
    table = np.array([[5, 1, 3]], dtype=np.int32)
    o, lse = O.full_attention("gqa", "f32", q, (k, v), table, [11], bs, 0.5, D)
    for h in range(Hkv * G):
        assert np.allclose(o[0, h], h // G, atol=1e-12), h


def check_mla_value_is_latent_prefix():
    """MLA V = first Dv dims of the cached row; rope dims only enter scores."""
    rng = np.random.default_rng(18)
    bs, N, Dqk, Dv = 4, 5, 10, 6
    cache = rng.standard_normal((N, bs, Dqk)).astype(np.float32)
    table = np.array([[4, 2, 0]], dtype=np.int32)
    q = rng.standard_normal((1, 3, Dqk)).astype(np.float32)
    L = 10
    o, lse = O.full_attention("mla", "f32", q, (cache,), table, [L], bs, 0.8, Dv)
    rows = np.stack([cache[table[0, t // bs], t % bs] for t in range(L)]).astype(np.float64)
    eo, el = _brute_attention(q[0].astype(np.float64).tolist(), rows.tolist(),
                              rows[:, :Dv].tolist(), 0.8)
    assert np.allclose(o[0], eo, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[0], el, rtol=1e-13)


def check_sharded_equals_full():
    """The DCP result (plan, partials, merge) equals unsharded attention."""
    from workloads import workload, make_host_inputs
    wl = workload("gqa-tiny")
    inp = make_host_inputs(wl)
    args = (wl.kind, wl.dtype, inp["q"], (inp["k_cache"], inp["v_cache"]), inp["block_table"])
    bounds, po, pl, o, lse = O.sharded_attention(*args, inp["seq_lens"], wl.num_shards,
                                                 wl.block_size, wl.softmax_scale, wl.head_dim_v)
    fo, fl = O.full_attention(*args, inp["seq_lens"], wl.block_size, wl.softmax_scale,
                              wl.head_dim_v)
    assert bounds[:, :, 1].tolist() == [[256, 512, 768, 1024]] * 2
    assert np.allclose(o, fo, rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, fl, rtol=1e-12, atol=1e-12)


def check_bf16_upcast():
    bits = np.array([0x3F80, 0xC000, 0x3F00, 0x0001, 0x7F7F, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 0.5, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, -0.0, 3.140625]
    got = O.bf16_bits_to_f64(bits)
    assert got.tolist() == want
    assert math.copysign(1.0, got[5]) == -1.0


# ------------------------------------------------------------------ several query tokens

def check_multi_hand_example():
    """Zero keys make every score 0, so a row's output is the mean of the values it may see:
    L = 3, two query tokens at positions 1 and 2, shards [0, 2) and [2, 3) (block size 1)."""
    v = np.array([[1.0, 0.0], [3.0, 6.0], [8.0, -3.0]])
    cache = np.zeros((3, 1, 4))
    cache[:, 0, :2] = v
    cache[:, 0, 2:] = 0.0
    q = np.ones((1, 2, 1, 4))
    q[..., :2] = 0.0                       # q . k = 0 for every row and token
    table = np.array([[2, 0, 1]], dtype=np.int32)
    paged = cache[[1, 2, 0]]               # page table[0, t] holds token t's row
    bounds = np.array([[[0, 2], [2, 3]]])
    po, pl = O.partial_attention_multi("mla", "f32", q.astype(np.float32),
                                       (paged.astype(np.float32),), table, bounds, 1, 0.5, 2)
    # token 0 (position 1) sees tokens 0, 1 in shard 0 and nothing in shard 1
    assert np.allclose(po[0, 0, 0, 0], [2.0, 3.0]) and math.isclose(pl[0, 0, 0, 0], math.log(2))
    assert np.all(po[0, 1, 0, 0] == 0.0) and np.isneginf(pl[0, 1, 0, 0])
    # token 1 (position 2) sees all three
    assert np.allclose(po[0, 1, 1, 0], [8.0, -3.0]) and math.isclose(pl[0, 1, 1, 0], 0.0,
                                                                     abs_tol=1e-15)
    o, lse = O.merge_lse(po.reshape(1, 2, 2, 2), pl.reshape(1, 2, 2))
    assert np.allclose(o[0, 1], [4.0, 1.0]) and math.isclose(lse[0, 1], math.log(3))
    assert np.allclose(o[0, 0], [2.0, 3.0])


def check_multi_rows_are_prefix_decodes():
    """Row j of a q_len-token step equals a one-token decode whose context ends at its own
    position, for every plan and both cache kinds; q_len = 1 is the one-token path."""
    from workloads import workload, make_host_inputs
    rng = np.random.default_rng(21)
    for name, lens, S, T in (("gqa-tiny", [40, 5], 3, 3), ("gqa-tiny", [17, 2], 2, 4),
                             ("gqa-tiny", [40, 9], 3, 20)):   # a chunk crossing shards
        wl = workload(name).replace(lengths=tuple(lens))
        inp = make_host_inputs(wl, lengths=lens)
        caches = (inp["k_cache"], inp["v_cache"])
        q = rng.standard_normal((wl.batch, T, wl.num_q_heads, wl.head_dim_qk)).astype(np.float32)
        _, _, _, o, lse = O.sharded_attention_multi("gqa", "f32", q, caches, inp["block_table"],
                                                    lens, S, wl.block_size, 0.2, wl.head_dim_v)
        for j in range(T):
            pre = [max(0, L - T + j + 1) for L in lens]
            fo, fl = O.full_attention("gqa", "f32", q[:, j], caches, inp["block_table"], pre,
                                      wl.block_size, 0.2, wl.head_dim_v)
            seen = np.array([p > 0 for p in pre])
            assert np.allclose(o[seen, j], fo[seen], rtol=1e-11, atol=1e-12)
            assert np.allclose(lse[seen, j], fl[seen], rtol=1e-12)
            assert np.all(o[~seen, j] == 0.0) and np.all(np.isneginf(lse[~seen, j]))
        one = O.partial_attention_multi("gqa", "f32", q[:, :1], caches, inp["block_table"],
                                        O.plan_shards(lens, S, wl.block_size), wl.block_size,
                                        0.2, wl.head_dim_v)
        ref = O.partial_attention("gqa", "f32", q[:, 0], caches, inp["block_table"],
                                  O.plan_shards(lens, S, wl.block_size), wl.block_size, 0.2,
                                  wl.head_dim_v)
        assert np.allclose(one[0][:, :, 0], ref[0], rtol=1e-13, atol=1e-14)
        assert np.array_equal(np.isneginf(one[1][:, :, 0]), np.isneginf(ref[1]))
        # a selection of query tokens computes exactly those rows and leaves the rest NaN
        bounds = O.plan_shards(lens, S, wl.block_size)
        full = O.partial_attention_multi("gqa", "f32", q, caches, inp["block_table"], bounds,
                                         wl.block_size, 0.2, wl.head_dim_v)
        pick = [0, T - 1]
        sub = O.partial_attention_multi("gqa", "f32", q, caches, inp["block_table"], bounds,
                                        wl.block_size, 0.2, wl.head_dim_v, tokens=pick)
        for a, b in zip(sub, full):
            assert np.array_equal(a[:, :, pick], b[:, :, pick])
            assert np.isnan(a[:, :, 1:T - 1]).all()


def check_multi_brute():
    """Pure-Python causal attention (exact sums) on a tiny MLA case, shards merged."""
    rng = np.random.default_rng(22)
    T, H, D, Dv, bs, L, S = 3, 2, 5, 3, 2, 7, 3
    rows = rng.standard_normal((L, D))
    table = np.array([[3, 0, 2, 1]], dtype=np.int32)
    cache = np.zeros((4, bs, D))
    for t in range(L):
        cache[table[0, t // bs], t % bs] = rows[t]
    q = rng.standard_normal((1, T, H, D))
    _, _, _, o, lse = O.sharded_attention_multi("mla", "f32", q.astype(np.float32),
                                                (cache.astype(np.float32),), table, [L], S, bs,
                                                0.7, Dv)
    r32 = cache.astype(np.float32).astype(np.float64)
    q32 = q.astype(np.float32).astype(np.float64)
    for j in range(T):
        seen = [r32[table[0, t // bs], t % bs] for t in range(L - T + j + 1)]
        for h in range(H):
            bo, bl = _brute_attention(q32[0, j, h:h + 1], np.stack(seen),
                                      np.stack(seen)[:, :Dv], 0.7)
            assert np.allclose(o[0, j, h], bo[0], rtol=1e-12, atol=1e-13)
            assert math.isclose(lse[0, j, h], bl[0], rel_tol=1e-13)


# ------------------------------------------------------------------ KV append

def check_append_example():
    """bs 4, table rows [2, 0, 3] and [1, 3, 0]: positions placed by hand."""
    bs, N, Hkv, D = 4, 4, 2, 3
    k = np.zeros((N, Hkv, bs, D))
    v = np.zeros((N, Hkv, bs, D))
    table = np.array([[2, 0, 3], [1, 3, 0]], dtype=np.int32)
    nk = np.arange(2 * Hkv * D, dtype=float).reshape(2, Hkv, D) + 1
    nv = -nk
    # request 0 holds 5 tokens: the sixth (position 5) goes to page 0, slot 1;
    # request 1 holds 8: position 8 is the first slot of its third page, 0.
    (k2, v2), owner = O.append_token("gqa", (k, v), (nk, nv), table, [5, 8], bs, 2)
    hit = sorted(map(tuple, np.argwhere(k2[..., 0] != 0).tolist()))
    assert hit == [(0, 0, 0), (0, 0, 1), (0, 1, 0), (0, 1, 1)], hit
    assert k2[0, :, 1].tolist() == nk[0].tolist() and v2[0, :, 1].tolist() == nv[0].tolist()
    assert k2[0, :, 0].tolist() == nk[1].tolist() and v2[0, :, 0].tolist() == nv[1].tolist()
    # 6 tokens on 2 shards of whole pages: [0, 4) and [4, 6) -> position 5 on shard 1;
    # 9 tokens: 3 pages, 2 per shard: [0, 8) and [8, 9) -> position 8 on shard 1.
    assert owner.tolist() == [1, 1]
    # A first token always lands on shard 0, page table[b, 0], slot 0.
    lat = np.zeros((N, bs, D))
    (lat2,), owner = O.append_token("mla", (lat,), (np.full((2, D), 7.0),), table, [0, 0], bs, 4)
    assert owner.tolist() == [0, 0]
    assert sorted(map(tuple, np.argwhere(lat2[..., 0] != 0).tolist())) == [(1, 0), (2, 0)]
    # Qiita's 200K tokens on 4 GPUs (0-50K, ..., 150K-200K): the token that completes the
    # 200K context is stored on the fourth GPU; token 100000 of a 100001-token request is on
    # the last shard of that request's own plan.
    big = np.zeros((1, 12500), dtype=np.int32)
    one = np.zeros((1, 1, D))
    _, owner = O.append_token("mla", (one[:, :1].repeat(16, 1),), (np.ones((1, D)),), big,
                              [199_999], 16, 4)
    assert owner.tolist() == [3]
    _, owner = O.append_token("mla", (one[:, :1].repeat(16, 1),), (np.ones((1, D)),), big,
                              [100_000], 16, 4)
    assert owner.tolist() == [3]


def check_append_replay():
    """Decoding token by token from empty pages rebuilds each request's dense history:
    the paged reader returns exactly the rows appended, pages outside the requests' tables
    stay untouched, and attention over the grown cache equals brute force on the history."""
    rng = np.random.default_rng(11)
    bs, N, Hkv, D, Dv, max_blocks = 4, 16, 2, 5, 3, 4
    lens = [13, 0, 7]
    B = len(lens)
    table = rng.permutation(N)[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    spare = sorted(set(range(N)) - set(table.ravel().tolist()))
    k = np.full((N, Hkv, bs, D), np.nan)
    v = np.full((N, Hkv, bs, Dv), np.nan)
    lat = np.full((N, bs, D), np.nan)
    hist_k = rng.standard_normal((B, max(lens), Hkv, D))
    hist_v = rng.standard_normal((B, max(lens), Hkv, Dv))
    for t in range(max(lens)):
        cur = [t if t < L else max_blocks * bs for L in lens]  # finished requests fall off
        (k, v), owner = O.append_token("gqa", (k, v), (hist_k[:, t], hist_v[:, t]), table, cur,
                                       bs, 3)
        (lat,), _ = O.append_token("mla", (lat,), (hist_k[:, t, 0],), table, cur, bs, 3)
        assert [o >= 0 for o in owner.tolist()] == [t < L for L in lens]
    for b, L in enumerate(lens):
        for g in range(Hkv):
            assert np.array_equal(O.gather_gqa(k, table, b, g, 0, L, bs), hist_k[b, :L, g])
            assert np.array_equal(O.gather_gqa(v, table, b, g, 0, L, bs), hist_v[b, :L, g])
        assert np.array_equal(O.gather_mla(lat, table, b, 0, L, bs), hist_k[b, :L, 0])
    assert np.isnan(k[spare]).all() and np.isnan(v[spare]).all() and np.isnan(lat[spare]).all()
    q = rng.standard_normal((Hkv, D))
    o, lse = O.attention(q, O.gather_gqa(k, table, 0, 1, 0, lens[0], bs),
                         O.gather_gqa(v, table, 0, 1, 0, lens[0], bs), 0.3)
    bo, blse = _brute_attention(q, hist_k[0, :lens[0], 1], hist_v[0, :lens[0], 1], 0.3)
    assert np.allclose(o, bo, rtol=1e-12, atol=1e-13) and np.allclose(lse, blse, rtol=1e-13)


def check_append_owner_brute(rng=None):
    """The owner is the shard whose brute-force range holds position L of an (L+1)-token
    request, and it is the last non-empty shard of that plan."""
    rng = rng or np.random.default_rng(12)
    cases = [(0, 1, 1), (0, 4, 16), (15, 4, 16), (16, 4, 16), (63, 8, 16), (64, 8, 16)]
    cases += [(int(rng.integers(0, 4000)), int(rng.integers(1, 17)),
               int(rng.choice([1, 3, 16, 64]))) for _ in range(200)]
    for L, S, bs in cases:
        pages = L // bs + 1
        table = np.zeros((1, pages), dtype=np.int32)
        _, owner = O.append_token("mla", (np.zeros((1, bs, 1)),), (np.ones((1, 1)),), table,
                                  [L], bs, S)
        ranges = _plan_brute(L + 1, S, bs)
        want = [s for s, (a, e) in enumerate(ranges) if a <= L < e]
        last = max(s for s, (a, e) in enumerate(ranges) if e > a)
        assert owner.tolist() == want == [last], (L, S, bs, owner, ranges)


def check_append_rejects():
    """Positions past the table row, negative lengths and page ids outside the pool store
    nothing and are reported with -1 / -2."""
    rng = np.random.default_rng(13)
    bs, N, Hkv, D = 4, 6, 1, 2
    k = rng.standard_normal((N, Hkv, bs, D))
    v = rng.standard_normal((N, Hkv, bs, D))
    table = np.array([[0, 1], [2, -1], [3, 6], [4, 5], [5, 4]], dtype=np.int32)
    new = (np.full((5, Hkv, D), 9.0), np.full((5, Hkv, D), 8.0))
    (k2, v2), owner = O.append_token("gqa", (k, v), new, table, [8, 4, -3, 11, 2], bs, 2)
    assert owner.tolist() == [-1, -2, -1, -1, 0]
    changed = sorted(map(tuple, np.argwhere((k2 != k).any(axis=-1)).tolist()))
    assert changed == [(5, 0, 2)], changed
    assert np.array_equal(k2[5, 0, 2], [9.0, 9.0]) and np.array_equal(v2[5, 0, 2], [8.0, 8.0])
    (k3, _), owner = O.append_token("gqa", (k, v), new, table, [0, 5, 4, 8, 8], bs, 2)
    assert owner.tolist() == [0, -2, -2, -1, -1]
    assert sorted(map(tuple, np.argwhere((k3 != k).any(axis=-1)).tolist())) == [(0, 0, 0)]


ALL_CHECKS = [
    check_bf16_upcast,
    check_plan_golden,
    check_plan_brute,
    check_gather_example,
    check_gather_fast_matches,
    check_gather_permutation_invariant,
    check_attention_brute,
    check_attention_library,
    check_attention_closed_forms,
    check_attention_laws,
    check_merge_partition_invariance,
    check_merge_associative_and_edge_cases,
    check_gqa_head_groups,
    check_mla_value_is_latent_prefix,
    check_sharded_equals_full,
    check_multi_hand_example,
    check_multi_rows_are_prefix_decodes,
    check_multi_brute,
    check_append_example,
    check_append_replay,
    check_append_owner_brute,
    check_append_rejects,
]
