"""GPU parity of the HIP path against the float64 oracle on small seeded inputs that span
several tiles, ragged tails, empty shards and every kernel family (through the C ABI)."""

import numpy as np
import pytest
import torch

import sequence_sharded_kv_amd as dcp
from gpu_helpers import (assert_close, assert_device_flags, host_inputs_of, oracle_full,
                         oracle_partials, run_fused, run_partial, say, shape_of, to_device)
from oracle import oracle as O
from workloads import make_host_inputs, workload

pytestmark = pytest.mark.gpu

# name, workload, lengths, overrides
CASES = [
    ("gqa-tiny", "gqa-tiny", None, {}),
    ("gqa-g16-bf16", "gqa-g16", [1, 700, 3001], dict(batch=3)),
    ("gqa-g16-bf16-S5", "gqa-g16", [4097, 33, 1000, 16], dict(batch=4, num_shards=5)),
    ("gqa-g8-planted20", "gqa-long", [5000, 2600], dict(batch=2)),
    ("gqa-g8-planted100", "gqa-long", [3000, 777], dict(batch=2, plant_score=100.0)),
    ("gqa-g4-d64-bf16", "gqa-g16", [900, 65], dict(batch=2, num_q_heads=16, head_dim_qk=64,
                                                  head_dim_v=64)),
    ("gqa-mqa-d128-bf16", "gqa-g16", [333, 1200], dict(batch=2, num_q_heads=4, num_kv_heads=4)),
    ("gqa-g16-f32-valu", "gqa-g16", [1500, 40], dict(batch=2, dtype="f32")),
    ("gqa-g16-d256-bf16-valu", "gqa-g16", [600, 129], dict(batch=2, head_dim_qk=256,
                                                          head_dim_v=256)),
    ("mla-64h", "mla-64h-b512", [1, 63, 64, 2000], dict(batch=4)),
    ("mla-64h-long", "mla-64h-b512", [9000, 4100], dict(batch=2)),
    ("mla-128h", "mla-128h", [3000, 777], dict(batch=2)),
    ("mla-32h", "mla-64h-b512", [1000, 2049, 5], dict(batch=3, num_q_heads=32)),
    ("mla-16h", "mla-64h-b512", [513, 70], dict(batch=2, num_q_heads=16)),
    ("mla-64h-bs16", "mla-64h-b512", [1000, 300], dict(batch=2, block_size=16)),
    # requests of length 0 (every shard empty) beside non-empty ones, and a batch of only
    # empty requests (no pages at all: every worker idle)
    ("gqa-g16-empty-requests", "gqa-g16", [0, 100, 0], dict(batch=3)),
    ("mla-64h-empty-requests", "mla-64h-b512", [0, 70, 0], dict(batch=3)),
    ("mla-64h-all-empty", "mla-64h-b512", [0, 0], dict(batch=2)),
    ("gqa-g16-all-empty", "gqa-g16", [0, 0], dict(batch=2)),
    # block size 1 (a tile spans 32 pages) and a non-power-of-two block size
    ("mla-64h-bs1", "mla-64h-b512", [200, 33], dict(batch=2, block_size=1)),
    ("gqa-g16-bs24", "gqa-g16", [500, 49], dict(batch=2, block_size=24)),
    ("mla-64h-bs48", "mla-64h-b512", [700, 97], dict(batch=2, block_size=48)),
    # output sizes that take the combine pass's one-thread-per-value instance (64 requests x
    # 64 heads x 512 dims): 16 shards (two batches of shards), and fewer pages than workers
    # (the pieces of a unit found through its pages' owners)
    ("mla-64h-b64-S16", "mla-64h-b512", [100 + 13 * i for i in range(64)],
     dict(batch=64, num_shards=16)),
    ("mla-64h-b64-few-pages", "mla-64h-b512", [20 + (7 * i) % 41 for i in range(64)],
     dict(batch=64, block_size=16, num_shards=2)),
]


def _setup(name, wl_name, lengths, over):
    wl = workload(wl_name).replace(**over)
    if lengths is not None and wl.length_law == "fixed":
        wl = wl.replace(lengths=tuple(lengths))
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    hin = host_inputs_of(wl, inp)
    return wl, host, inp, hin


@pytest.mark.parametrize("name,wl_name,lengths,over", CASES, ids=[c[0] for c in CASES])
def test_partials_merge_and_fused_match_oracle(name, wl_name, lengths, over):
    say(f"[gpu] parity case {name}")
    wl, host, inp, hin = _setup(name, wl_name, lengths, over)
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, wl.block_size)
    bounds = torch.from_numpy(bounds_np).cuda()
    po, pl, ws = run_partial(wl, inp, bounds)
    out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32,
                      device="cuda")
    out_lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device="cuda")
    dcp.dcp_merge_lse(po, pl, out, out_lse)
    fo, fl, _ = run_fused(wl, inp, bounds, ws=ws)
    torch.cuda.synchronize()
    assert_device_flags(ws, wl)
    ro, rl = oracle_partials(wl, hin, bounds_np)
    assert_close(po.cpu().numpy(), pl.cpu().numpy(), ro, rl, wl.dtype, f"{name} partials")
    fo_ref, fl_ref = oracle_full(wl, hin)
    assert_close(out.cpu().numpy(), out_lse.cpu().numpy(), fo_ref, fl_ref, wl.dtype,
                 f"{name} merged")
    assert_close(fo.cpu().numpy(), fl.cpu().numpy(), fo_ref, fl_ref, wl.dtype, f"{name} fused")


@pytest.mark.parametrize("wl_name,over,lengths", [
    ("gqa-tiny", {}, None),
    ("gqa-g16", dict(batch=2), [1000, 37]),
    ("mla-64h-b512", dict(batch=2), [700, 65]),
])
def test_debug_gather_is_bit_exact(wl_name, over, lengths):
    say(f"[gpu] gather {wl_name}")
    wl = workload(wl_name).replace(**over)
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, wl.block_size)
    bounds = torch.from_numpy(bounds_np).cuda()
    sh = shape_of(wl, inp)
    cache = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    hcache = host["kv_cache"] if wl.kind == "mla" else host["k_cache"]
    for b in range(wl.batch):
        for s in range(wl.num_shards):
            a, e = int(bounds_np[b, s, 0]), int(bounds_np[b, s, 1])
            for g in range(wl.num_kv_heads):
                dst = torch.zeros((max(e - a, 1), wl.head_dim_qk), dtype=cache.dtype, device="cuda")
                dcp.dcp_debug_gather_shard(sh, cache, inp["block_table"], bounds, b, s, g, dst)
                got = dst.view(torch.int16 if cache.dtype == torch.bfloat16 else torch.int32)
                got = got.cpu().numpy()[: e - a]
                if wl.kind == "mla":
                    want = O.gather_mla(hcache, host["block_table"], b, a, e, wl.block_size)
                else:
                    want = O.gather_gqa(hcache, host["block_table"], b, g, a, e, wl.block_size)
                assert got.tobytes() == np.ascontiguousarray(want).tobytes(), (b, s, g)


def test_device_plan_matches_oracle_plan():
    """The device plan, bit for bit, against oracle.plan_shards (and the host plan)."""
    say("[gpu] device plan")
    rng = np.random.default_rng(1)
    for S, bs in ((1, 16), (4, 16), (8, 64), (16, 16), (7, 1), (3, 48)):
        lens = rng.integers(0, 1_100_000, size=37).astype(np.int32)
        lens[:5] = [0, 1, bs, bs + 1, S * bs - 1]
        d = dcp.dcp_plan_shards_device(torch.from_numpy(lens).cuda(), S, bs).cpu().numpy()
        want = O.plan_shards(lens, S, bs)
        assert d.dtype == np.int32 and d.shape == want.shape
        assert np.array_equal(d.astype(np.int64), want), (S, bs)
        assert np.array_equal(d, dcp.dcp_plan_shards(lens, S, bs))


@pytest.mark.parametrize("wl_name,over,lengths", [
    ("gqa-g16", dict(batch=3), [2000, 1, 517]),
    ("mla-64h-b512", dict(batch=3), [1500, 64, 3]),
    ("gqa-tiny", {}, None),
])
def test_any_partition_merges_to_full_attention(wl_name, over, lengths):
    """Caller-chosen contiguous partitions (unaligned cuts, one-token and empty shards)."""
    say(f"[gpu] partitions {wl_name}")
    wl = workload(wl_name).replace(**over)
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    hin = host_inputs_of(wl, inp)
    want_o, want_l = oracle_full(wl, hin)
    rng = np.random.default_rng(5)
    lens = host["seq_lens"]
    for S in (1, 3, 9):
        bounds_np = np.zeros((wl.batch, S, 2), np.int32)
        for b in range(wl.batch):
            cuts = np.sort(rng.integers(0, lens[b] + 1, size=S - 1))
            if S > 2 and lens[b] > 2:
                cuts[0] = cuts[1] = min(cuts[1], lens[b] - 1)  # an empty shard
            edges = [0] + cuts.tolist() + [int(lens[b])]
            bounds_np[b, :, 0], bounds_np[b, :, 1] = edges[:-1], edges[1:]
        bounds = torch.from_numpy(bounds_np).cuda()
        fo, fl, ws = run_fused(wl, inp, bounds, num_shards=S)
        torch.cuda.synchronize()
        assert_close(fo.cpu().numpy(), fl.cpu().numpy(), want_o, want_l, wl.dtype,
                     f"{wl_name} S={S}")
        po, pl, _ = run_partial(wl, inp, bounds, num_shards=S, ws=ws)
        ro, rl = oracle_partials(wl, hin, bounds_np)
        assert_close(po.cpu().numpy(), pl.cpu().numpy(), ro, rl, wl.dtype, f"{wl_name} S={S} parts")


@pytest.mark.parametrize("wl_name,over,lengths", [
    ("mla-64h-b512", dict(batch=3), [1000, 77, 4097]),                   # wave pairs
    ("mla-64h-b512", dict(batch=2, num_q_heads=32), [900, 61]),         # 16 rows per wave
    ("mla-128h", dict(batch=2), [2000, 45]),                            # 8-wave pairs
    ("mla-64h-b512", dict(batch=2, block_size=16), [500, 77]),         # tiles over 2 pages
    ("mla-64h-b512", dict(batch=2, num_q_heads=32, block_size=16), [300, 50]),
    ("mla-128h", dict(batch=2, block_size=16), [400, 39]),
    ("gqa-g16", dict(batch=3), [1000, 77, 3001]),                       # 32-row kernel
    ("gqa-g16", dict(batch=2, num_q_heads=16, head_dim_qk=64, head_dim_v=64),
     [700, 45]),                                                        # 16-row kernel
    ("gqa-g16", dict(batch=2, dtype="f32"), [700, 45]),                 # VALU kernel
], ids=["mla-64h", "mla-32h", "mla-128h", "mla-64h-bs16", "mla-32h-bs16", "mla-128h-bs16",
        "gqa-g16", "gqa-g4-d64", "gqa-g16-f32"])
def test_unused_slots_past_the_context_stay_out_of_the_output(wl_name, over, lengths):
    """A page's slots past the context end may hold anything in a real cache. Filled with NaN
    here, they must not reach the output: masked tokens get weight 0, and 0 * NaN would
    poison the value product if a kernel copied those slots."""
    say(f"[gpu] NaN past the context: {wl_name} {over} {lengths}")
    wl = workload(wl_name).replace(**over)
    if wl.length_law == "fixed":
        wl = wl.replace(lengths=tuple(lengths))
    host = make_host_inputs(wl, lengths=lengths)
    inp = to_device(wl, host)
    bt = host["block_table"]
    names = ("kv_cache",) if wl.kind == "mla" else ("k_cache", "v_cache")
    filled = 0
    for b, L in enumerate(lengths):
        tail = L % wl.block_size
        if tail == 0:
            continue
        page = int(bt[b, L // wl.block_size])
        for n in names:
            if wl.kind == "mla":
                inp[n][page, tail:, :] = float("nan")
            else:
                inp[n][page, :, tail:, :] = float("nan")
        filled += wl.block_size - tail
    assert filled > 0
    hin = host_inputs_of(wl, inp)
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, wl.block_size)
    bounds = torch.from_numpy(bounds_np).cuda()
    fo, fl, ws = run_fused(wl, inp, bounds)
    torch.cuda.synchronize()
    assert_device_flags(ws, wl)
    o, l = fo.cpu().numpy(), fl.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(l).all()
    fo_ref, fl_ref = oracle_full(wl, hin)
    assert_close(o, l, fo_ref, fl_ref, wl.dtype, f"{wl_name} NaN past the context")


def test_workspace_reuse_poison_and_determinism():
    say("[gpu] workspace reuse")
    wl = workload("mla-64h-b512").replace(batch=3)
    host = make_host_inputs(wl, lengths=[3000, 700, 45])
    inp = to_device(wl, host)
    bounds = torch.from_numpy(dcp.dcp_plan_shards(host["seq_lens"], 8, 64)).cuda()
    out, lse, ws = run_fused(wl, inp, bounds)
    ref = out.clone(), lse.clone()
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for i in range(20):
        if i % 2 == 0:
            ws.fill_(0xFF)  # NaN bytes everywhere in the workspace
        run_fused(wl, inp, bounds, ws=ws, out=out, out_lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])
    g = workload("gqa-g16").replace(batch=2)
    gh = make_host_inputs(g, lengths=[5000, 300])
    gi = to_device(g, gh)
    gb = torch.from_numpy(dcp.dcp_plan_shards(gh["seq_lens"], 2, 16)).cuda()
    o1, l1, gws = run_fused(g, gi, gb)
    gws.fill_(0xFF)
    o2, l2, _ = run_fused(g, gi, gb, ws=gws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_invalid_device_values_are_flagged_not_faulted():
    """A block id outside the pool and a bound past the table are handled on the device
    (masked / clamped) and reported through the workspace flag word."""
    say("[gpu] device-side validation")
    for wl_name, over, lengths in (("gqa-g16", dict(batch=2), [100, 200]),
                                   ("mla-64h-b512", dict(batch=2), [100, 200]),
                                   ("gqa-tiny", {}, None)):
        wl = workload(wl_name).replace(**over)
        host = make_host_inputs(wl, lengths=lengths)
        inp = to_device(wl, host)
        bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, wl.block_size)
        bt = inp["block_table"].clone()
        bt[1, 0] = int(host["num_blocks"]) + 7
        inp2 = dict(inp, block_table=bt)
        bounds = torch.from_numpy(bounds_np).cuda()
        out, lse, ws = run_fused(wl, inp2, bounds)
        torch.cuda.synchronize()
        assert dcp.dcp_read_device_flags(ws) & 2
        hin = host_inputs_of(wl, inp)
        fo, fl = oracle_full(wl, hin, seqs=[0])
        assert_close(out.cpu().numpy()[:1], lse.cpu().numpy()[:1], fo[:1], fl[:1], wl.dtype,
                     f"{wl_name} untouched sequence")
        assert torch.isfinite(out).all()
        big = bounds_np.copy()
        big[0, -1, 1] = 10 ** 9
        out, lse, ws = run_fused(wl, inp, torch.from_numpy(big).cuda())
        torch.cuda.synchronize()
        assert dcp.dcp_read_device_flags(ws) & 1
        assert torch.isfinite(out).all()
