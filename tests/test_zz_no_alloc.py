"""dcp_decode_attn_noalloc (the workspace is the library's static device scratch) against
dcp_decode_attn with a caller-allocated workspace, through the C ABI: two calls in a row,
the second on a smaller input, so that the scratch still holds the first call's contents;
each result is compared element by element with the workspace entry point on the same
inputs, and with the float64 oracle."""

import pytest
import torch

import sequence_sharded_kv_amd as dcp
from gpu_helpers import (assert_close, device_caches, host_inputs_of, oracle_full, run_fused,
                         say, shape_of, to_device)
from workloads import make_host_inputs, workload

pytestmark = pytest.mark.gpu

# (workload, lengths, overrides): a larger call, then a smaller one
SEQUENCES = [
    ("mla", [("mla-64h-b512", [3000, 777, 64], dict(batch=3)),
             ("mla-64h-b512", [150], dict(batch=1))]),
    ("gqa", [("gqa-g16", [4000, 1, 900, 2500], dict(batch=4)),
             ("gqa-g16", [300, 17], dict(batch=2))]),
    ("mla-128h", [("mla-128h", [2100, 900], dict(batch=2)),
                  ("mla-64h-b512", [70], dict(batch=1, num_q_heads=32))]),
]


def _noalloc(wl, inp, bounds):
    sh = shape_of(wl, inp)
    out = torch.full((wl.batch, wl.num_q_heads, wl.head_dim_v), float("nan"),
                     dtype=torch.float32, device="cuda")
    out_lse = torch.full((wl.batch, wl.num_q_heads), float("nan"), dtype=torch.float32,
                         device="cuda")
    k, v = device_caches(wl, inp)
    dcp.dcp_decode_attn_noalloc(sh, inp["q"], k, v, inp["block_table"], bounds, out, out_lse)
    return out, out_lse


@pytest.mark.parametrize("name,calls", SEQUENCES, ids=[s[0] for s in SEQUENCES])
def test_noalloc_matches_workspace_entry_point(name, calls):
    for i, (wl_name, lengths, over) in enumerate(calls):
        say(f"[gpu] noalloc {name} call {i}: {wl_name} {lengths}")
        wl = workload(wl_name).replace(**over)
        if wl.length_law == "fixed":
            wl = wl.replace(lengths=tuple(lengths))
        host = make_host_inputs(wl, lengths=lengths)
        inp = to_device(wl, host)
        assert dcp.dcp_workspace_bytes(shape_of(wl, inp)) <= dcp.DCP_NOALLOC_SCRATCH_BYTES
        bounds_np = dcp.dcp_plan_shards(host["seq_lens"], wl.num_shards, wl.block_size)
        bounds = torch.from_numpy(bounds_np).cuda()
        no, nl = _noalloc(wl, inp, bounds)
        wo, wl_lse, _ = run_fused(wl, inp, bounds)
        no2, nl2 = _noalloc(wl, inp, bounds)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: equal bit for bit, and deterministic
        assert torch.equal(no, wo) and torch.equal(nl, wl_lse), f"{name} call {i}"
        assert torch.equal(no, no2) and torch.equal(nl, nl2), f"{name} call {i} repeat"
        fo, fl = oracle_full(wl, host_inputs_of(wl, inp))
        assert_close(no.cpu().numpy(), nl.cpu().numpy(), fo, fl, wl.dtype,
                     f"{name} call {i} noalloc")
