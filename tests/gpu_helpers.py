"""Shared pieces of the GPU tests: running the library on seeded inputs and comparing with
the float64 oracle at the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

import sequence_sharded_kv_amd as dcp
from oracle import oracle as O

# (max-abs on O, relative L2 on O, max-abs on LSE): bf16 KV with fp32 accumulation, and fp32.
TOL = {"bf16": (2e-3, 1e-3, 2e-3), "f32": (1e-4, 1e-5, 1e-4)}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def assert_device_flags(ws, wl) -> None:
    """No error bit in the workspace's device flag word. Bit 3 (a worker raised a row's
    reference maximum and rescaled it) is expected only where the workload plants high-score
    keys: a planted key met past a worker's first tile raises the reference."""
    import sequence_sharded_kv_amd as dcp
    flags = dcp.dcp_read_device_flags(ws)
    allowed = (0, 8) if getattr(wl, "plants_per_head", 0) else (0,)
    assert flags in allowed, flags


def host_view(t):
    """numpy copy of a device tensor: bf16 as uint16 bit patterns, others as-is."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def shape_of(wl, inp, num_shards=None):
    bt = inp["block_table"]
    return dcp.make_shape(wl.kind, wl.dtype, wl.batch, wl.num_q_heads, wl.num_kv_heads,
                          wl.head_dim_qk, wl.head_dim_v, wl.block_size, int(bt.shape[1]),
                          int(inp["num_blocks"]), num_shards or wl.num_shards, wl.softmax_scale)


def device_caches(wl, inp):
    if wl.kind == "mla":
        return inp["kv_cache"], None
    return inp["k_cache"], inp["v_cache"]


def to_device(wl, host, device="cuda"):
    """Device tensors from make_host_inputs output."""
    out = {"num_blocks": host["num_blocks"]}
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    for k in ("q", "k_cache", "v_cache", "kv_cache"):
        if k in host:
            out[k] = dev(host[k])
            assert out[k].dtype == tdt
    out["block_table"] = torch.from_numpy(host["block_table"]).to(device)
    out["seq_lens"] = torch.from_numpy(host["seq_lens"]).to(device)
    return out


def host_inputs_of(wl, inp, seqs=None):
    """Host copies for the oracle. With `seqs`, only the pages those sequences use are kept
    (the block table is renumbered to the copied pages)."""
    bt = inp["block_table_host"] if "block_table_host" in inp else inp["block_table"].cpu().numpy()
    lens = inp["seq_lens_host"] if "seq_lens_host" in inp else inp["seq_lens"].cpu().numpy()
    q = host_view(inp["q"])
    names = ("kv_cache",) if wl.kind == "mla" else ("k_cache", "v_cache")
    if seqs is None:
        caches = tuple(host_view(inp[n]) for n in names)
        return q, caches, bt, lens
    pages = []
    for b in seqs:
        n = -(-int(lens[b]) // wl.block_size)
        pages.append(bt[b, :n])
    pages = np.concatenate(pages) if pages else np.zeros(0, np.int32)
    uniq = np.unique(pages)
    remap = {int(p): i for i, p in enumerate(uniq)}
    idx = torch.from_numpy(uniq.astype(np.int64)).to(inp["q"].device)
    caches = tuple(host_view(inp[n].index_select(0, idx)) for n in names)
    bt2 = np.full_like(bt, -1)
    for b in seqs:
        n = -(-int(lens[b]) // wl.block_size)
        bt2[b, :n] = [remap[int(p)] for p in bt[b, :n]]
    return q, caches, bt2, lens


def run_partial(wl, inp, bounds, num_shards=None, ws=None):
    sh = shape_of(wl, inp, num_shards)
    B, S, Hq, Dv = wl.batch, sh.num_shards, wl.num_q_heads, wl.head_dim_v
    dev = inp["q"].device
    po = torch.empty((B, S, Hq, Dv), dtype=torch.float32, device=dev)
    pl = torch.empty((B, S, Hq), dtype=torch.float32, device=dev)
    if ws is None:
        ws = dcp.alloc_workspace(sh, dev)
    k, v = device_caches(wl, inp)
    dcp.dcp_decode_attn_partial(sh, inp["q"], k, v, inp["block_table"], bounds, po, pl, ws)
    return po, pl, ws


def run_fused(wl, inp, bounds, num_shards=None, ws=None, out=None, out_lse=None):
    sh = shape_of(wl, inp, num_shards)
    dev = inp["q"].device
    if ws is None:
        ws = dcp.alloc_workspace(sh, dev)
    if out is None:
        out = torch.empty((wl.batch, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32, device=dev)
        out_lse = torch.empty((wl.batch, wl.num_q_heads), dtype=torch.float32, device=dev)
    k, v = device_caches(wl, inp)
    dcp.dcp_decode_attn(sh, inp["q"], k, v, inp["block_table"], bounds, ws, out, out_lse)
    return out, out_lse, ws


def oracle_partials(wl, host, bounds_np, seqs=None):
    q, caches, bt, _ = host
    return O.partial_attention(wl.kind, wl.dtype, q, caches, bt, np.asarray(bounds_np, np.int64),
                               wl.block_size, wl.softmax_scale, wl.head_dim_v, seqs)


def oracle_full(wl, host, seqs=None):
    q, caches, bt, lens = host
    return O.full_attention(wl.kind, wl.dtype, q, caches, bt, lens, wl.block_size,
                            wl.softmax_scale, wl.head_dim_v, seqs)


def assert_close(got_o, got_lse, want_o, want_lse, dtype, what):
    """O: max-abs and relative L2 within TOL; LSE: max-abs. Rows whose oracle LSE is -inf
    (empty ranges) must be exactly O = 0 and LSE = -inf."""
    atol, rl2, latol = TOL[dtype]
    got_o = np.asarray(got_o, np.float64)
    got_lse = np.asarray(got_lse, np.float64)
    empty = np.isneginf(want_lse)
    if empty.any():
        assert np.all(got_o[empty] == 0.0), f"{what}: empty rows not zero"
        assert np.all(np.isneginf(got_lse[empty])), f"{what}: empty rows' LSE not -inf"
    keep = ~empty
    if not keep.any():
        return 0.0, 0.0
    a, b = got_o[keep], want_o[keep]
    assert np.all(np.isfinite(a)), f"{what}: non-finite output"
    err = float(np.max(np.abs(a - b)))
    rel = float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
    lerr = float(np.max(np.abs(got_lse[keep] - want_lse[keep])))
    say(f"  {what}: max-abs {err:.3e} rel-L2 {rel:.3e} lse max-abs {lerr:.3e}")
    assert err <= atol, f"{what}: max-abs {err} > {atol}"
    assert rel <= rl2, f"{what}: rel-L2 {rel} > {rl2}"
    assert lerr <= latol, f"{what}: LSE max-abs {lerr} > {latol}"
    return err, rel
