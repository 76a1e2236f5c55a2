"""The seeded input generators (CPU only)."""

import math

import numpy as np
import torch

from workloads import (WORKLOADS, bf16_bits_from_f32, draw_block_table, draw_lengths,
                       make_host_inputs, workload)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0,
                                  65504.0, 1e-30], dtype=np.float32)])
    ours = bf16_bits_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_block_table_is_a_partition_of_the_pool():
    ss = np.random.SeedSequence(5)
    lens = np.array([0, 1, 16, 17, 1000, 64])
    table, n = draw_block_table(lens, 16, ss)
    need = [-(-int(L) // 16) for L in lens]
    assert n == sum(need)
    used = np.concatenate([table[b, :k] for b, k in enumerate(need)])
    assert sorted(used.tolist()) == list(range(n))
    for b, k in enumerate(need):
        assert np.all(table[b, k:] == -1)


def test_lengths_follow_their_laws():
    wl = workload("mla-64h-b512")
    lens = draw_lengths(wl, np.random.SeedSequence(1004).spawn(5)[0])
    assert lens.shape == (512,) and lens.min() >= 1
    med = float(np.median(lens))
    assert 55_000 < med < 80_000
    p5, p95 = np.percentile(lens, [5, 95])
    assert 15_000 < p5 < 35_000 and 130_000 < p95 < 230_000
    wl3 = workload("mla-128h")
    lens3 = draw_lengths(wl3, np.random.SeedSequence(1003).spawn(5)[0])
    assert lens3.max() <= 131072
    wl2 = workload("gqa-g16")
    lens2 = draw_lengths(wl2, np.random.SeedSequence(1002).spawn(5)[0])
    assert lens2.min() >= 8192 and lens2.max() <= 32768


def test_host_inputs_are_reproducible_and_shaped():
    wl = workload("gqa-tiny")
    a = make_host_inputs(wl)
    b = make_host_inputs(wl)
    for k in ("q", "k_cache", "v_cache", "block_table", "seq_lens"):
        assert np.array_equal(a[k], b[k])
    assert a["k_cache"].shape == (128, 2, 16, 64) and a["k_cache"].dtype == np.float32
    assert sorted(a["block_table"].ravel().tolist()) == list(range(128))
    mla = workload("mla-64h-b512").replace(batch=3)
    m = make_host_inputs(mla, lengths=[5, 130, 64])
    assert m["kv_cache"].dtype == np.uint16 and m["kv_cache"].shape[1:] == (64, 576)
    lat = (m["kv_cache"][..., :512].astype(np.uint32) << 16).view(np.float32)
    rope = (m["kv_cache"][..., 512:].astype(np.uint32) << 16).view(np.float32)
    assert 0.45 < lat.std() < 0.55 and 0.9 < rope.std() < 1.1


def test_planted_keys_reach_their_score():
    wl = workload("gqa-long").replace(batch=2, lengths=(3000, 5000))
    inp = make_host_inputs(wl)
    q = (inp["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = (inp["k_cache"].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    G = wl.group_size
    assert len(inp["plants"]) == 2 * wl.num_kv_heads * 3
    for b, g, t in inp["plants"]:
        row = k[inp["block_table"][b, t // 16], g, t % 16]
        s = wl.softmax_scale * (q[b, g * G:(g + 1) * G] @ row)
        assert abs(s.mean() - 20.0) < 0.5, (b, g, t, s.mean())


def test_every_workload_is_consistent():
    for name, wl in WORKLOADS.items():
        assert wl.num_q_heads % wl.num_kv_heads == 0, name
        assert wl.head_dim_v <= wl.head_dim_qk
        assert math.isfinite(wl.softmax_scale) and wl.softmax_scale > 0
