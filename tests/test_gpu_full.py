"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
sampled sequences (shortest, longest and random ones) are checked element by element
against the float64 oracle; properties that hold at any size are checked on every output."""

import numpy as np
import pytest
import torch

import sequence_sharded_kv_amd as dcp
from gpu_helpers import (assert_close, host_inputs_of, oracle_partials, run_fused, run_partial,
                         say)
from oracle import oracle as O
from workloads import make_device_inputs, workload

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.mark.parametrize("name,nrand", [("gqa-g16", 2), ("gqa-long", 0), ("mla-128h", 1),
                                        ("mla-64h-b512", 1)])
def test_full_size_sampled_parity(name, nrand):
    wl = workload(name)
    say(f"[gpu] full-size {name}: drawing inputs")
    inp = make_device_inputs(wl, "cuda")
    lens = inp["seq_lens_host"]
    bounds_np = dcp.dcp_plan_shards(lens, wl.num_shards, wl.block_size)
    bounds = torch.from_numpy(bounds_np).cuda()
    say(f"[gpu] full-size {name}: fused + partial, {int(lens.sum())} tokens")
    out, out_lse, ws = run_fused(wl, inp, bounds)
    po, pl, _ = run_partial(wl, inp, bounds, ws=ws)
    torch.cuda.synchronize()
    assert dcp.dcp_read_device_flags(ws) == 0
    # properties over every output: finite, and O is a convex combination of value rows
    assert torch.isfinite(out).all() and torch.isfinite(out_lse).all()
    vals = inp["kv_cache"][..., : wl.head_dim_v] if wl.kind == "mla" else inp["v_cache"]
    vmax = max(abs(float(vals.amax().float())), abs(float(vals.amin().float())))
    assert float(out.abs().amax()) <= vmax * (1 + 1e-6)
    rng = np.random.default_rng(99)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens))}
                  | set(int(x) for x in rng.choice(wl.batch, size=nrand, replace=False)))
    say(f"[gpu] full-size {name}: oracle on sequences {seqs} (lengths {[int(lens[s]) for s in seqs]})")
    host = host_inputs_of(wl, inp, seqs)
    ro, rl = oracle_partials(wl, host, bounds_np, seqs)
    mo, ml = O.merge_lse(ro[seqs], rl[seqs])
    assert_close(po.cpu().numpy()[seqs], pl.cpu().numpy()[seqs], ro[seqs], rl[seqs], wl.dtype,
                 f"{name} partials")
    assert_close(out.cpu().numpy()[seqs], out_lse.cpu().numpy()[seqs], mo, ml, wl.dtype,
                 f"{name} fused")
    del inp, out, po, pl, ws
    torch.cuda.empty_cache()
