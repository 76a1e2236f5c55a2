"""GPU parity of several query tokens per request (causal rows) against the float64 oracle:
partials, the merge and the fused call, for MLA and both GQA kernels, with row counts that
fit one unit, that need several row groups and that leave padding rows; prefill chunks of
33-200 tokens; requests shorter than q_len; and q_len = 1 through the multi-token calls
against the one-token calls."""

import numpy as np
import pytest
import torch

import sequence_sharded_kv_amd as dcp
from gpu_helpers import (assert_close, assert_device_flags, host_inputs_of, run_partial, say,
                         shape_of, to_device)
from oracle import oracle as O
from workloads import make_host_inputs, make_queries, workload

pytestmark = pytest.mark.gpu


def _q_device(wl, qh):
    if qh.dtype == np.uint16:
        return torch.from_numpy(qh.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(qh).cuda()


# name, workload, lengths, q_len, overrides
CASES = [
    ("mla-64h-t2", "mla-64h-b512", [2000, 1, 700], 2, dict(batch=3)),
    # 129 to 192 rows: two passes, 128 rows through the 128-row kernel and the rest through a
    # smaller unit, for the partial and the fused call
    ("mla-64h-t3-split", "mla-64h-b512", [1500, 64, 2], 3, dict(batch=3)),
    ("mla-32h-t6-split", "mla-64h-b512", [800, 90], 6, dict(batch=2, num_q_heads=32)),
    # second pass of 32 rows (the 16-rows-per-wave kernel), requests shorter than q_len
    ("mla-32h-t5-split-32", "mla-64h-b512", [700, 130, 3], 5, dict(batch=3, num_q_heads=32)),
    ("mla-16h-t10-split", "mla-64h-b512", [500, 9], 10, dict(batch=2, num_q_heads=16)),
    ("mla-16h-t8", "mla-64h-b512", [900, 8, 3], 8, dict(batch=3, num_q_heads=16)),
    ("mla-128h-t2", "mla-128h", [1200, 33], 2, dict(batch=2)),
    ("mla-32h-t3-padding", "mla-64h-b512", [600, 97], 3, dict(batch=2, num_q_heads=32)),
    ("mla-64h-t4-bs1", "mla-64h-b512", [150, 5], 4, dict(batch=2, block_size=1)),
    # 64 rows per unit (the wave-pair kernel) from several query tokens: a wave's partner
    # holds the other token's rows, or padding rows (16 heads x 3 tokens = 48 of 64)
    ("mla-32h-t2-pair", "mla-64h-b512", [1300, 45], 2, dict(batch=2, num_q_heads=32)),
    ("mla-16h-t3-pair-padding", "mla-64h-b512", [800, 130, 2], 3, dict(batch=3,
                                                                      num_q_heads=16)),
    ("mla-16h-t4-pair-bs16", "mla-64h-b512", [700, 64], 4, dict(batch=2, num_q_heads=16,
                                                               block_size=16)),
    # 128 rows per unit (the 8-wave pair kernel): 16 heads x 5 tokens = 80 of 128 rows, two
    # pages per tile, and 32 heads x 3 tokens with a non-power-of-two page
    ("mla-16h-t5-pair8-padding", "mla-64h-b512", [900, 70, 3], 5, dict(batch=3,
                                                                       num_q_heads=16)),
    ("mla-128h-pair8-bs16", "mla-128h", [1100, 40], 1, dict(batch=2, block_size=16)),
    ("mla-32h-t3-pair8-bs48", "mla-64h-b512", [1000, 95], 3, dict(batch=2, num_q_heads=32,
                                                                block_size=48)),
    ("gqa-g16-t2", "gqa-g16", [3000, 1, 100], 2, dict(batch=3)),
    ("gqa-g4-d64-t4", "gqa-g16", [900, 3], 4, dict(batch=2, num_q_heads=16, head_dim_qk=64,
                                                    head_dim_v=64)),
    ("gqa-g8-t3-S16", "gqa-long", [5000, 40], 3, dict(batch=2, plants_per_head=0)),
    ("gqa-f32-valu-t2", "gqa-g16", [1100, 2], 2, dict(batch=2, dtype="f32")),
    ("gqa-d256-valu-t3", "gqa-g16", [700, 70], 3, dict(batch=2, head_dim_qk=256,
                                                      head_dim_v=256)),
    ("gqa-g16-t5-bs24", "gqa-g16", [500, 49], 5, dict(batch=2, block_size=24)),
    # 48 rows per KV head: one 2-wave unit of 64 rows; 160 rows: one 8-wave unit of 256 rows
    # on 64-token tiles, 96 of them padding
    ("gqa-g16-t3-64rows", "gqa-g16", [900, 70], 3, dict(batch=2)),
    ("gqa-g16-t10-256rows", "gqa-g16", [700, 33], 10, dict(batch=2)),
    # 64-token tiles across pages: 24-token pages (non-power-of-two) and one-token pages (a
    # tile spans 64 pages, the most one lookup of page ids holds)
    ("gqa-g16-t10-bs24", "gqa-g16", [600, 45], 10, dict(batch=2, block_size=24)),
    ("gqa-g16-t12-bs1", "gqa-g16", [300, 20], 12, dict(batch=2, block_size=1)),
    # prefill chunks: many row groups per shard, chunks that cross shard boundaries, and a
    # request shorter than its chunk
    ("mla-64h-chunk64", "mla-64h-b512", [1500, 300], 64, dict(batch=2, num_shards=4)),
    ("mla-16h-chunk96", "mla-64h-b512", [900, 40], 96, dict(batch=2, num_q_heads=16)),
    ("mla-128h-chunk33", "mla-128h", [700, 90], 33, dict(batch=2)),
    ("gqa-g16-chunk48", "gqa-g16", [1000, 120], 48, dict(batch=2)),
    ("gqa-g8-chunk200-S16", "gqa-long", [5000, 600], 200, dict(batch=2, plants_per_head=0)),
    ("gqa-f32-valu-chunk40", "gqa-g16", [400, 30], 40, dict(batch=2, dtype="f32")),
]


@pytest.mark.parametrize("name,wl_name,lengths,T,over", CASES, ids=[c[0] for c in CASES])
def test_multi_token_partials_and_fused_match_oracle(name, wl_name, lengths, T, over):
    say(f"[gpu] multi-token case {name} (q_len {T})")
    wl = workload(wl_name).replace(**over)
    if wl.length_law == "fixed":
        wl = wl.replace(lengths=tuple(lengths))
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    qh = make_queries(wl, T)
    q = _q_device(wl, qh)
    sh = shape_of(wl, inp)
    B, S, Hq, Dv = wl.batch, wl.num_shards, wl.num_q_heads, wl.head_dim_v
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], S, wl.block_size)
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda", T)
    k = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    v = None if wl.kind == "mla" else inp["v_cache"]
    po = torch.empty((B, S, T, Hq, Dv), dtype=torch.float32, device="cuda")
    pl = torch.empty((B, S, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi_partial(sh, T, q, k, v, inp["block_table"], bounds, po, pl, ws)
    out = torch.empty((B, T, Hq, Dv), dtype=torch.float32, device="cuda")
    out_lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi(sh, T, q, k, v, inp["block_table"], bounds, ws, out, out_lse)
    mo = torch.empty_like(out)
    ml = torch.empty_like(out_lse)
    dcp.dcp_merge_lse(po.view(B, S, T * Hq, Dv), pl.view(B, S, T * Hq), mo.view(B, T * Hq, Dv),
                      ml.view(B, T * Hq))
    torch.cuda.synchronize()
    assert_device_flags(ws, wl)
    _, caches, bt, _ = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention_multi(wl.kind, wl.dtype, qh, caches, bt,
                                       np.asarray(bounds_np, np.int64), wl.block_size,
                                       wl.softmax_scale, Dv)
    assert_close(po.cpu().numpy().reshape(B, S, T * Hq, Dv), pl.cpu().numpy().reshape(B, S, T * Hq),
                 ro.reshape(B, S, T * Hq, Dv), rl.reshape(B, S, T * Hq), wl.dtype,
                 f"{name} partials")
    fo, fl = O.merge_lse(ro.reshape(B, S, T * Hq, Dv), rl.reshape(B, S, T * Hq))
    assert_close(out.cpu().numpy().reshape(B, T * Hq, Dv), out_lse.cpu().numpy().reshape(B, T * Hq),
                 fo, fl, wl.dtype, f"{name} fused")
    assert_close(mo.cpu().numpy().reshape(B, T * Hq, Dv), ml.cpu().numpy().reshape(B, T * Hq),
                 fo, fl, wl.dtype, f"{name} merged")
    # a request shorter than q_len: its first tokens see nothing at all
    for b, L in enumerate(lengths):
        for j in range(T):
            if L - T + j + 1 <= 0:
                assert torch.all(out[b, j] == 0) and torch.all(torch.isneginf(out_lse[b, j]))


# prefill chunks of the sizes bench.py --q-len times (512 and 4096 tokens) on short contexts:
# name, workload, lengths, q_len, overrides
CHUNKS = [
    ("mla-64h-chunk512", "mla-64h-b512", [1100, 700], 512, dict(batch=2)),
    ("mla-64h-chunk4096", "mla-64h-b512", [4500], 4096, dict(batch=1, num_shards=4)),
    ("gqa-g16-chunk512", "gqa-g16", [1300, 600], 512, dict(batch=2)),
    ("gqa-g16-chunk4096", "gqa-g16", [4400], 4096, dict(batch=1)),
]


@pytest.mark.parametrize("name,wl_name,lengths,T,over", CHUNKS, ids=[c[0] for c in CHUNKS])
def test_prefill_chunk_sampled_tokens_match_oracle(name, wl_name, lengths, T, over):
    """Every shard and head of 16 query tokens of the chunk (the first two, the middle, the
    last two and 11 seeded others), partials and the fused call, against the oracle computed
    for those tokens alone; every output is finite."""
    say(f"[gpu] prefill chunk {name} (q_len {T})")
    wl = workload(wl_name).replace(**over)
    if wl.length_law == "fixed":
        wl = wl.replace(lengths=tuple(lengths))
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    qh = make_queries(wl, T)
    q = _q_device(wl, qh)
    sh = shape_of(wl, inp)
    B, S, Hq, Dv = wl.batch, wl.num_shards, wl.num_q_heads, wl.head_dim_v
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], S, wl.block_size)
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda", T)
    k = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    v = None if wl.kind == "mla" else inp["v_cache"]
    po = torch.empty((B, S, T, Hq, Dv), dtype=torch.float32, device="cuda")
    pl = torch.empty((B, S, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi_partial(sh, T, q, k, v, inp["block_table"], bounds, po, pl, ws)
    out = torch.empty((B, T, Hq, Dv), dtype=torch.float32, device="cuda")
    out_lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi(sh, T, q, k, v, inp["block_table"], bounds, ws, out, out_lse)
    torch.cuda.synchronize()
    assert_device_flags(ws, wl)
    assert torch.isfinite(out).all() and torch.isfinite(po).all()
    rng = np.random.default_rng(5)
    pick = sorted({0, 1, T // 2, T - 2, T - 1} |
                  set(int(x) for x in rng.choice(T, size=11, replace=False)))
    _, caches, bt, _ = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention_multi(wl.kind, wl.dtype, qh, caches, bt,
                                       np.asarray(bounds_np, np.int64), wl.block_size,
                                       wl.softmax_scale, Dv, tokens=pick)
    ro, rl = ro[:, :, pick], rl[:, :, pick]
    n = len(pick)
    assert_close(po[:, :, pick].cpu().numpy().reshape(B, S, n * Hq, Dv),
                 pl[:, :, pick].cpu().numpy().reshape(B, S, n * Hq),
                 ro.reshape(B, S, n * Hq, Dv), rl.reshape(B, S, n * Hq), wl.dtype,
                 f"{name} partials")
    fo, fl = O.merge_lse(ro.reshape(B, S, n * Hq, Dv), rl.reshape(B, S, n * Hq))
    assert_close(out[:, pick].cpu().numpy().reshape(B, n * Hq, Dv),
                 out_lse[:, pick].cpu().numpy().reshape(B, n * Hq), fo, fl, wl.dtype,
                 f"{name} fused")


@pytest.mark.parametrize("wl_name,over,lengths", [
    ("mla-64h-b512", dict(batch=3), [1000, 77, 1]),
    ("gqa-g16", dict(batch=3), [2000, 50, 0]),
])
def test_multi_with_one_token_equals_one_token_calls(wl_name, over, lengths):
    """q_len = 1 through the multi-token calls gives the one-token calls' bits."""
    say(f"[gpu] q_len 1 through the multi-token calls: {wl_name}")
    wl = workload(wl_name).replace(**over)
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    sh = shape_of(wl, inp)
    bounds = torch.from_numpy(dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards,
                                                  wl.block_size)).cuda()
    ws = dcp.alloc_workspace(sh, "cuda")
    k = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    v = None if wl.kind == "mla" else inp["v_cache"]
    o1 = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device="cuda")
    l1 = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn(sh, inp["q"], k, v, inp["block_table"], bounds, ws, o1, l1)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    dcp.dcp_decode_attn_multi(sh, 1, inp["q"], k, v, inp["block_table"], bounds, ws, o2, l2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("wl_name", ["mla-128h", "mla-64h-b512"])
def test_lazy_max_mla_handles_scores_that_outrun_the_first_tile(wl_name):
    """The MLA kernels for 64 and 128 query rows per unit take weights relative to each
    segment's first-tile maximum. Two keys planted mid-shard score about 90 (natural log
    units) above the rest: the workers that meet them raise the rows' reference and rescale
    their sums and accumulators in place (flag bit 3), and the result matches the oracle."""
    from workloads import bf16_bits_from_f32
    say(f"[gpu] lazy-max MLA kernel with planted high-score keys: {wl_name}")
    wl = workload(wl_name).replace(batch=2)
    lengths = [3000, 2000]
    host = make_host_inputs(wl, lengths=lengths)
    bs = wl.block_size
    q0 = (host["q"][0, 0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    c = 90.0 / (wl.softmax_scale * float(q0 @ q0))
    key = bf16_bits_from_f32((c * q0).astype(np.float32))
    # positions in the second half of their 64-token page: with this little work every
    # non-empty worker covers one page, so the plant is past each segment's first tile
    for t in (2536, 1330):
        host["kv_cache"][host["block_table"][0, t // bs], t % bs] = key
    inp = to_device(wl, host)
    sh = shape_of(wl, inp)
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, bs)
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32,
                      device="cuda")
    out_lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn(sh, inp["q"], inp["kv_cache"], None, inp["block_table"], bounds, ws, out,
                        out_lse)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) == 8
    hq, caches, bt, lens = host_inputs_of(wl, inp)
    fo, fl = O.full_attention("mla", wl.dtype, hq, caches, bt, lens, bs, wl.softmax_scale,
                              wl.head_dim_v)
    assert float(np.max(fl[0])) > 80.0
    assert_close(out.cpu().numpy(), out_lse.cpu().numpy(), fo, fl, wl.dtype, "planted high score")


def test_lazy_max_gqa_chunk_handles_scores_that_outrun_the_first_tile():
    """The GQA chunk kernel also weights each row against its first-tile maximum. Keys
    planted at four places in shard 1 of request 0 score about 90 (natural log units) above
    the rest for one query row of a 48-token chunk: the workers that meet one past their first
    tile raise that row's reference and rescale its sum and accumulator (flag bit 3), and the
    partials and the fused result match the oracle."""
    from workloads import bf16_bits_from_f32
    say("[gpu] lazy-max GQA chunk kernel with planted high-score keys")
    wl = workload("gqa-g16").replace(batch=2)
    lengths = [3000, 1000]
    T = 48
    host = make_host_inputs(wl, lengths=lengths)
    qh = make_queries(wl, T)
    bs = wl.block_size
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, bs)
    # query token 5, head 3 (KV head 0) of request 0
    qv = (qh[0, 5, 3].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    c = 90.0 / (wl.softmax_scale * float(qv @ qv))
    key = bf16_bits_from_f32((c * qv).astype(np.float32))
    start = int(bounds_np[0, 1, 0])
    for k in range(4):
        t = start + (10 + 20 * k) * bs + 5
        assert t < lengths[0] - T
        host["k_cache"][host["block_table"][0, t // bs], 0, t % bs] = key
    inp = to_device(wl, host)
    q = _q_device(wl, qh)
    sh = shape_of(wl, inp)
    B, S, Hq, Dv = wl.batch, wl.num_shards, wl.num_q_heads, wl.head_dim_v
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda", T)
    po = torch.empty((B, S, T, Hq, Dv), dtype=torch.float32, device="cuda")
    pl = torch.empty((B, S, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi_partial(sh, T, q, inp["k_cache"], inp["v_cache"],
                                      inp["block_table"], bounds, po, pl, ws)
    out = torch.empty((B, T, Hq, Dv), dtype=torch.float32, device="cuda")
    out_lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi(sh, T, q, inp["k_cache"], inp["v_cache"], inp["block_table"],
                              bounds, ws, out, out_lse)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) == 8
    _, caches, bt, _ = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention_multi(wl.kind, wl.dtype, qh, caches, bt,
                                       np.asarray(bounds_np, np.int64), bs, wl.softmax_scale, Dv)
    assert float(np.max(rl[0, 1, 5, 3])) > 80.0
    assert_close(po.cpu().numpy().reshape(B, S, T * Hq, Dv), pl.cpu().numpy().reshape(B, S, T * Hq),
                 ro.reshape(B, S, T * Hq, Dv), rl.reshape(B, S, T * Hq), wl.dtype,
                 "chunk planted partials")
    fo, fl = O.merge_lse(ro.reshape(B, S, T * Hq, Dv), rl.reshape(B, S, T * Hq))
    assert_close(out.cpu().numpy().reshape(B, T * Hq, Dv), out_lse.cpu().numpy().reshape(B, T * Hq),
                 fo, fl, wl.dtype, "chunk planted fused")


@pytest.mark.parametrize("case", ["huge-value", "tiny-values"])
def test_fp16_value_kernel_recomputes_what_fp16_cannot_hold(case):
    """128 query rows per unit take the value product in fp16. A latent value of 70000
    (beyond fp16's 65504) in one request, or a request whose latent rows are all scaled
    below 2^-10, sends the workers that meet them to the bf16 kernel (flag bit 2); the
    result matches the oracle."""
    from workloads import bf16_bits_from_f32
    say(f"[gpu] fp16 value range: {case}")
    wl = workload("mla-128h").replace(batch=2)
    lengths = [1500, 700]
    host = make_host_inputs(wl, lengths=lengths)
    bs = wl.block_size
    cache = host["kv_cache"]
    if case == "huge-value":
        t = 900
        row = (cache[host["block_table"][0, t // bs], t % bs].astype(np.uint32) << 16) \
            .view(np.float32).copy()
        row[5] = 70000.0
        cache[host["block_table"][0, t // bs], t % bs] = bf16_bits_from_f32(row)
    else:
        pages = host["block_table"][1, : -(-lengths[1] // bs)]
        vals = (cache[pages].astype(np.uint32) << 16).view(np.float32)
        cache[pages] = bf16_bits_from_f32((vals * 2.0 ** -12).astype(np.float32))
    inp = to_device(wl, host)
    sh = shape_of(wl, inp)
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, bs)
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32,
                      device="cuda")
    out_lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn(sh, inp["q"], inp["kv_cache"], None, inp["block_table"], bounds, ws, out,
                        out_lse)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) & 4
    hq, caches, bt, lens = host_inputs_of(wl, inp)
    fo, fl = O.full_attention("mla", wl.dtype, hq, caches, bt, lens, bs, wl.softmax_scale,
                              wl.head_dim_v)
    if case == "tiny-values":
        assert_close(out.cpu().numpy(), out_lse.cpu().numpy(), fo, fl, wl.dtype, case)
    else:
        # outputs and LSEs reach about 7e4 and 5e3 here: the bounds are relative to them
        got, lse = out.cpu().numpy().astype(np.float64), out_lse.cpu().numpy().astype(np.float64)
        scale = max(1.0, float(np.abs(fo).max()))
        assert np.all(np.isfinite(got))
        assert float(np.abs(got - fo).max()) <= 2e-3 * scale
        assert float(np.linalg.norm(got - fo) / np.linalg.norm(fo)) <= 1e-3
        assert float(np.abs(lse - fl).max()) <= 1e-3 * max(1.0, float(np.abs(fl).max()))


def test_ring_kernel_raises_the_reference_several_times_in_one_segment():
    """64 query rows per unit (the ring kernel). In one shard, keys scoring about 90, 180,
    270 and 360 above the rest for head 0 sit in four consecutive 32-token tiles from the
    second tile of a page on. A worker covers six or more pages here, so whichever page
    boundary splits them, one segment meets at least two of them after its first tile and
    raises that row's reference twice or more. In the other request a high key for head 9
    raises another row. The rescaled sums and accumulators match the oracle."""
    from workloads import bf16_bits_from_f32
    say("[gpu] ring kernel: repeated reference raises in one segment")
    wl = workload("mla-64h-b512").replace(batch=2)
    lengths = [60000, 50000]
    host = make_host_inputs(wl, lengths=lengths)
    bs = wl.block_size

    def plant(b, t, head, target):
        qh = (host["q"][b, head].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        c = target / (wl.softmax_scale * float(qh @ qh))
        host["kv_cache"][host["block_table"][b, t // bs], t % bs] = \
            bf16_bits_from_f32((c * qh).astype(np.float32))

    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, bs)
    lo, hi = (int(x) for x in bounds_np[0, 1])
    base = lo + 10 * bs + 32
    assert base + 128 < hi
    for k, target in enumerate((90.0, 180.0, 270.0, 360.0)):
        plant(0, base + 32 * k, 0, target)
    plant(1, 3500, 9, 90.0)
    inp = to_device(wl, host)
    sh = shape_of(wl, inp)
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda")
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32,
                      device="cuda")
    out_lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn(sh, inp["q"], inp["kv_cache"], None, inp["block_table"], bounds, ws, out,
                        out_lse)
    po, pl, _ = run_partial(wl, inp, bounds, ws=ws)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) == 8
    hq, caches, bt, lens = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention("mla", wl.dtype, hq, caches, bt, np.asarray(bounds_np, np.int64),
                                 bs, wl.softmax_scale, wl.head_dim_v)
    assert float(rl[0, 1, 0]) > 350.0 and float(rl[1].max()) > 80.0
    assert_close(po.cpu().numpy(), pl.cpu().numpy(), ro, rl, wl.dtype, "raised, partials")
    fo, fl = O.merge_lse(ro, rl)
    assert_close(out.cpu().numpy(), out_lse.cpu().numpy(), fo, fl, wl.dtype, "raised, fused")


@pytest.mark.parametrize("wl_name,over,lengths,T", [
    ("gqa-g16", dict(batch=2), [300, 200], 4),       # 64 rows per KV head: gqa_chunk_kernel
    ("mla-64h-b512", dict(batch=2), [300, 200], 1),  # 64 rows: mla_ring_kernel
    ("mla-64h-b512", dict(batch=2), [300, 200], 2),  # 128 rows: mla_pair16_kernel
    ("mla-128h", dict(batch=2), [300, 200], 1),      # 128 heads: mla_pair16_kernel
])
def test_multi_row_kernels_flag_invalid_device_values(wl_name, over, lengths, T):
    """The kernels for many rows per KV tile mask a block id outside the pool and clamp a
    bound past the table like the others: flags set, other requests exact, output finite."""
    say(f"[gpu] device-side validation, {wl_name} q_len {T}")
    wl = workload(wl_name).replace(**over)
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    qh = make_queries(wl, T)
    q = _q_device(wl, qh)
    sh = shape_of(wl, inp)
    B, S, Hq, Dv = wl.batch, wl.num_shards, wl.num_q_heads, wl.head_dim_v
    k = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    v = None if wl.kind == "mla" else inp["v_cache"]
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], S, wl.block_size)
    ws = dcp.alloc_workspace(sh, "cuda", T)
    out = torch.empty((B, T, Hq, Dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    bt = inp["block_table"].clone()
    bt[1, 0] = int(host["num_blocks"]) + 7
    dcp.dcp_decode_attn_multi(sh, T, q, k, v, bt, torch.from_numpy(bounds_np).cuda(), ws, out, lse)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) & 2
    assert torch.isfinite(out).all()
    _, caches, hbt, _ = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention_multi(wl.kind, wl.dtype, qh, caches, hbt,
                                       np.asarray(bounds_np, np.int64), wl.block_size,
                                       wl.softmax_scale, Dv, seqs=[0])
    fo, fl = O.merge_lse(ro[:1].reshape(1, S, T * Hq, Dv), rl[:1].reshape(1, S, T * Hq))
    assert_close(out.cpu().numpy()[:1].reshape(1, T * Hq, Dv),
                 lse.cpu().numpy()[:1].reshape(1, T * Hq), fo, fl, wl.dtype,
                 f"{wl_name} untouched request")
    big = bounds_np.copy()
    big[0, -1, 1] = 10 ** 9
    dcp.dcp_decode_attn_multi(sh, T, q, k, v, inp["block_table"], torch.from_numpy(big).cuda(), ws,
                              out, lse)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) & 1
    assert torch.isfinite(out).all()


def test_two_pass_call_keeps_the_first_pass_flags():
    """64 heads x 3 tokens run as a 128-row pass (fp16 value product) and a 64-row pass. With
    one request's latent rows scaled below 2^-10, the first pass recomputes its workers in
    bf16 (flag bit 2); the second pass must not clear that bit, and the outputs match the
    oracle."""
    from workloads import bf16_bits_from_f32
    say("[gpu] two-pass call keeps the first pass's flags")
    T = 3
    wl = workload("mla-64h-b512").replace(batch=2)
    lengths = [900, 400]
    host = make_host_inputs(wl, lengths=lengths)
    bs = wl.block_size
    cache = host["kv_cache"]
    pages = host["block_table"][1, : -(-lengths[1] // bs)]
    vals = (cache[pages].astype(np.uint32) << 16).view(np.float32)
    cache[pages] = bf16_bits_from_f32((vals * 2.0 ** -12).astype(np.float32))
    inp = to_device(wl, host)
    sh = shape_of(wl, inp)
    B, S, Hq, Dv = wl.batch, wl.num_shards, wl.num_q_heads, wl.head_dim_v
    qh = make_queries(wl, T)
    q = _q_device(wl, qh)
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], S, bs)
    bounds = torch.from_numpy(bounds_np).cuda()
    ws = dcp.alloc_workspace(sh, "cuda", T)
    out = torch.empty((B, T, Hq, Dv), dtype=torch.float32, device="cuda")
    out_lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    dcp.dcp_decode_attn_multi(sh, T, q, inp["kv_cache"], None, inp["block_table"], bounds, ws,
                              out, out_lse)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) & 4
    _, caches, bt, _ = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention_multi(wl.kind, wl.dtype, qh, caches, bt,
                                       np.asarray(bounds_np, np.int64), bs, wl.softmax_scale, Dv)
    fo, fl = O.merge_lse(ro.reshape(B, S, T * Hq, Dv), rl.reshape(B, S, T * Hq))
    assert_close(out.cpu().numpy().reshape(B, T * Hq, Dv), out_lse.cpu().numpy().reshape(B, T * Hq),
                 fo, fl, wl.dtype, "two-pass tiny values")
