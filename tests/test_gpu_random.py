"""Seeded random shapes through the fused call, against the float64 oracle: every kernel
family (MLA 16/32/64/128 heads; GQA MFMA, chunk and VALU kernels), one to nine shards,
block sizes from 1 to 64, empty and ragged requests, one to 40 query tokens. The list is
drawn once from a fixed seed, so every run checks the same cases."""

import numpy as np
import pytest
import torch

import sequence_sharded_kv_amd as dcp
from gpu_helpers import (assert_close, assert_device_flags, host_inputs_of, say, shape_of,
                         to_device)
from oracle import oracle as O
from workloads import make_host_inputs, make_queries, workload

pytestmark = pytest.mark.gpu


def _draw_cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        kind = "mla" if i % 2 == 0 else "gqa"
        B = int(rng.integers(1, 4))
        S = int(rng.integers(1, 10))
        bs = int(rng.choice([1, 7, 16, 32, 64]))
        T = int(rng.choice([1, 1, 2, 3, 8, 40]))
        lens = [int(x) for x in rng.integers(0, 600, size=B)]
        if rng.random() < 0.3:
            lens[0] = 0
        if kind == "mla":
            over = dict(batch=B, num_q_heads=int(rng.choice([16, 32, 64, 128])), num_shards=S,
                        block_size=bs, length_law="fixed", lengths=tuple(lens))
            base = "mla-64h-b512"
        else:
            G = int(rng.choice([1, 2, 4, 8, 16]))
            Hkv = int(rng.choice([1, 2, 4]))
            D = int(rng.choice([64, 128, 128, 256]))
            dtype = str(rng.choice(["bf16", "bf16", "f32"]))
            over = dict(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim_qk=D,
                        head_dim_v=D, dtype=dtype, num_shards=S, block_size=bs,
                        softmax_scale=float(D) ** -0.5, length_law="fixed", lengths=tuple(lens),
                        plants_per_head=0)
            base = "gqa-g16"
        cases.append((f"{i:02d}-{kind}", base, over, T))
    return cases


CASES = _draw_cases()


@pytest.mark.parametrize("name,base,over,T", CASES, ids=[c[0] for c in CASES])
def test_random_shape_matches_oracle(name, base, over, T):
    wl = workload(base).replace(**over)
    say(f"[gpu] random case {name}: B {wl.batch} Hq {wl.num_q_heads} Hkv {wl.num_kv_heads} "
        f"D {wl.head_dim_qk} {wl.dtype} S {wl.num_shards} bs {wl.block_size} q_len {T} "
        f"lengths {list(wl.lengths)}")
    host = make_host_inputs(wl, lengths=list(wl.lengths))
    inp = to_device(wl, host)
    qh = make_queries(wl, T, seed=7000 + int(name[:2]))
    q = (torch.from_numpy(qh.view(np.int16)).cuda().view(torch.bfloat16) if qh.dtype == np.uint16
         else torch.from_numpy(qh).cuda())
    sh = shape_of(wl, inp)
    B, S, Hq, Dv = wl.batch, wl.num_shards, wl.num_q_heads, wl.head_dim_v
    bounds_np = dcp.dcp_plan_shards(host["seq_lens"], S, wl.block_size)
    ws = dcp.alloc_workspace(sh, "cuda", T)
    out = torch.empty((B, T, Hq, Dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, T, Hq), dtype=torch.float32, device="cuda")
    k = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    v = None if wl.kind == "mla" else inp["v_cache"]
    dcp.dcp_decode_attn_multi(sh, T, q, k, v, inp["block_table"],
                              torch.from_numpy(bounds_np).cuda(), ws, out, lse)
    torch.cuda.synchronize()
    assert_device_flags(ws, wl)
    _, caches, bt, _ = host_inputs_of(wl, inp)
    ro, rl = O.partial_attention_multi(wl.kind, wl.dtype, qh, caches, bt,
                                       np.asarray(bounds_np, np.int64), wl.block_size,
                                       wl.softmax_scale, Dv)
    fo, fl = O.merge_lse(ro.reshape(B, S, T * Hq, Dv), rl.reshape(B, S, T * Hq))
    assert_close(out.cpu().numpy().reshape(B, T * Hq, Dv), lse.cpu().numpy().reshape(B, T * Hq),
                 fo, fl, wl.dtype, name)
