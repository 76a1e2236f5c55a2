#!/usr/bin/env python
"""Benchmark of sequence-sharded paged decode attention + LSE merge on one MI355X.

One step = one dcp_decode_attn call (per-shard partials over the paged KV cache, kept in the
reused workspace, then the LSE merge) for the whole batch of one layer, with Q and the KV
cache already resident in HBM. The default workload is the agent-style MLA decode batch:
512 requests, 64 query heads sharing one 576-dim latent (value = first 512 dims), bf16,
lognormal contexts with median 67K tokens, 64-token pages, 8 contiguous shards per request.

Prints one JSON line: the whole-step algorithmic HBM throughput (TB/s) as `value`, decode
steps/s, the dominant kernel's roofline (its own launch time from HIP events recorded by
the library on the launch stream) and the float64 CPU oracle timed on a bounded sample.
With --q-len T > 1 a step scores T query tokens per request (dcp_decode_attn_multi, causal
rows) over the same cache; the KV bytes are still counted once. T > 16 is a prefill chunk
(e.g. --workload mla-prefill --q-len 512): `value` and the roofline are then algorithmic
TFLOP/s against the dense bf16 MFMA peak.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "mla": ["k_mla_mfma.hip", "mla_common.h", "device_common.h", "dcp_internal.h"],
    "mla-ring": ["k_mla_ring.hip", "mla_common.h", "device_common.h", "dcp_internal.h"],
    "mla-split": ["k_mla_pair16.hip", "k_mla_ring.hip", "mla_common.h", "device_common.h",
                  "dcp_internal.h"],
    "mla-pair": ["k_mla_pair16.hip", "mla_common.h", "device_common.h", "dcp_internal.h"],
    "gqa-mfma": ["k_gqa_mfma.hip", "device_common.h", "dcp_internal.h"],
    "gqa-chunk": ["k_gqa_chunk.hip", "device_common.h", "dcp_internal.h"],
    "gqa-valu": ["k_gqa_valu.hip", "device_common.h", "dcp_internal.h"],
}
KERNEL_NAMES = {"mla": "mla_mfma_kernel", "mla-ring": "mla_ring_kernel",
                "mla-pair": "mla_pair16_kernel",
                "mla-split": "mla_pair16_kernel + mla_ring_kernel",
                "gqa-mfma": "gqa_mfma_kernel", "gqa-chunk": "gqa_chunk_kernel",
                "gqa-valu": "gqa_valu_kernel"}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="mla-64h-b512")
    p.add_argument("--q-len", type=int, default=1,
                   help="query tokens per request (speculative / MTP decode); 1 = plain decode")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--plant-high-keys", type=float, default=0.0, metavar="FRACTION",
                   help="MLA only: in this fraction of the requests (seeded), overwrite one "
                        "latent row in the middle of a random shard with a key that scores "
                        "90 (natural log units) above the rest for one head, so that the "
                        "workers meeting it outrun their first tile's maximum")
    p.add_argument("--ceiling-gib", type=float, default=4.0,
                   help="buffer size of the HBM streaming-read ceiling measured in the same run "
                        "(0 skips it)")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--calibration-copy-gib", type=float, default=0.0,
                   help="before timing, run one fp32 x1.0 elementwise pass over this many GiB "
                        "(reference dispatch for counter calibration)")
    p.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                        "script and print the traffic JSON")
    p.add_argument("--pmc-calibration-gib", type=float, default=1.0)
    p.add_argument("--summarize-mfma", metavar="MFMA_DIR",
                   help="summarise a rocprofv3 --pmc run (MfmaUtil MfmaFlopsBF16 "
                        "SQ_INSTS_VALU_MFMA_BF16) of this script and print the MFMA JSON")
    return p.parse_args()


# ------------------------------------------------------------------ byte model

def kernel_family(wl, q_len=1):
    if wl.kind == "mla":
        # units of 64 query rows take the 12-wave ring kernel, of 128 the 8-wave fp16 pair
        # kernel, smaller units the 16-rows-per-wave kernel
        rows = q_len * wl.num_q_heads
        if 128 < rows <= 192:
            # two passes: 128 rows through the pair kernel, the rest (at most 64) through the
            # ring kernel
            return "mla-split"
        return "mla-pair" if rows > 64 else "mla-ring" if rows > 32 else "mla"
    g = wl.num_q_heads // wl.num_kv_heads
    if wl.dtype == "bf16" and g <= 16 and wl.head_dim_qk == 128:
        return "gqa-chunk"   # units of 32 to 128 query rows of one KV head share each K/V tile
    if wl.dtype == "bf16" and g <= 16 and wl.head_dim_qk == 64:
        return "gqa-mfma"
    return "gqa-valu"


def byte_model(wl, lens, q_len=1):
    """Algorithmic bytes of one step: what the method must move at least once (the KV once,
    whatever the number of query tokens)."""
    esz = 2 if wl.dtype == "bf16" else 4
    tokens = int(np.sum(lens))
    if wl.kind == "mla":
        kv = tokens * wl.head_dim_qk * esz                      # V shares the latent bytes
    else:
        kv = tokens * wl.num_kv_heads * wl.head_dim_qk * esz * 2
    rows = q_len * wl.num_q_heads
    q = wl.batch * rows * wl.head_dim_qk * esz
    table = int(np.sum(-(-np.asarray(lens, np.int64) // wl.block_size))) * 4
    part = wl.batch * wl.num_shards * rows * (wl.head_dim_v + 1) * 4
    out = wl.batch * rows * (wl.head_dim_v + 1) * 4
    return {"kv": kv, "q": q, "table": table, "partials_rw": 2 * part, "out": out,
            "step": kv + q + table + 2 * part + out,
            "partial_kernel": kv + q + table + part, "tokens": tokens}


def flop_model(wl, lens, q_len):
    """Algorithmic flops of a step of q_len causal query tokens per request: every (row, visible
    token) pair costs 2 Dqk (score) + 2 Dv (value) flops."""
    per = 2 * wl.head_dim_qk + 2 * wl.head_dim_v
    vis = 0
    for L in np.asarray(lens, np.int64):
        j = np.arange(q_len, dtype=np.int64)
        vis += int(np.maximum(0, int(L) - q_len + j + 1).sum())
    return vis * wl.num_q_heads * per


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16


def sources_sha(family):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "sequence_sharded_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(workload):
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def mfma_file(workload):
    return os.path.join(PROFILES, f"mfma_{workload}.json")


def load_traffic(workload, family, path=None):
    path = path or traffic_file(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sources_sha256") != sources_sha(family):
        return None  # the kernel changed since the counters were taken
    return t


# ------------------------------------------------------------------ rocprofv3 counters

def _read_counter_csv(d, counter):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((int(r.get("Dispatch_Id", 0)), r.get("Kernel_Name", ""),
                                 float(r["Counter_Value"])))
    rows.sort()
    return rows


def summarize_pmc(fetch_dir, write_dir, workload, family, calib_gib):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the dominant kernel, scaled by what the
    same counters read for the fp32 elementwise reference pass over calib_gib GiB."""
    out = {"workload": workload, "kernel": KERNEL_NAMES[family],
           "kernel_sources_sha256": sources_sha(family)}
    ref_bytes = calib_gib * (1 << 30)
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _read_counter_csv(d, name)
        ker = [(i, v) for i, k, v in rows if KERNEL_NAMES[family] in k]
        if not ker:
            raise SystemExit(f"{name}: no dispatches of {KERNEL_NAMES[family]} in {d}")
        # the reference pass is the last elementwise dispatch before the first attention step
        # (the input generators before it are elementwise kernels too)
        ref = [v for i, k, v in rows if "elementwise" in k.lower() and i < ker[0][0]]
        if not ref or not 0.25 * ref_bytes <= ref[-1] * 1024 <= 4 * ref_bytes:
            raise SystemExit(f"{name}: no reference pass of about {calib_gib} GiB before the "
                             f"first {KERNEL_NAMES[family]} dispatch in {d}")
        ker = [v for _, v in ker]
        scale = ref_bytes / (ref[-1] * 1024.0)
        out[name.lower() + "_kib_raw_mean"] = float(np.mean(ker))
        out[name.lower() + "_calibration_scale"] = scale
        out[name.lower() + "_bytes_per_launch"] = float(np.mean(ker)) * 1024.0 * scale
        out[name.lower() + "_dispatches"] = len(ker)
    out["traffic_bytes_per_launch"] = out["fetch_size_bytes_per_launch"] + \
        out["write_size_bytes_per_launch"]
    return out


def summarize_mfma(d, workload, family, wl):
    """MFMA counters of the dominant kernel, averaged over its dispatches: MfmaUtil (percent of
    the GPU-active cycles during which the SIMDs' matrix units are busy, summed over SIMDs),
    the matrix operations issued (MfmaFlops over every type, or MfmaFlopsBF16 in older runs;
    512 per MOPS count) and the bf16 (+ fp16) MFMA instruction count. Issued flops include any
    second value product of split weights and padding rows."""
    out = {"workload": workload, "kernel": KERNEL_NAMES[family],
           "kernel_sources_sha256": sources_sha(family)}

    def mean_of(name, required=True):
        ker = [v for _, k, v in _read_counter_csv(d, name) if KERNEL_NAMES[family] in k]
        if not ker:
            if required:
                raise SystemExit(f"{name}: no dispatches of {KERNEL_NAMES[family]} in {d}")
            return None, 0
        return float(np.mean(ker)), len(ker)

    out["mfma_busy_pct"], out["mfma_busy_pct_dispatches"] = mean_of("MfmaUtil")
    flops, nd = mean_of("MfmaFlops", required=False)
    if flops is None:
        flops, nd = mean_of("MfmaFlopsBF16")
    out["mfma_flops_per_launch"], out["mfma_flops_dispatches"] = flops, nd
    inst, nd = mean_of("SQ_INSTS_VALU_MFMA_BF16")
    f16, _ = mean_of("SQ_INSTS_VALU_MFMA_F16", required=False)
    if f16 is not None:
        out["mfma_instructions_bf16_per_launch"] = inst
        out["mfma_instructions_f16_per_launch"] = f16
        inst += f16
    out["mfma_instructions_per_launch"], out["mfma_instructions_dispatches"] = inst, nd
    out["flops_per_instruction"] = out["mfma_flops_per_launch"] / out["mfma_instructions_per_launch"]
    return out


# ------------------------------------------------------------------ planted keys

def plant_high_keys(wl, inp, bounds_np, q_dev, frac, seed=11, score=90.0):
    """Overwrite one latent row in the middle of a random shard of round(frac * batch)
    seeded requests with c * q[b, j, h] (bf16), c chosen so that head h of query token j
    scores `score` above zero on it. Returns the number of requests planted."""
    import torch
    rng = np.random.default_rng(seed)
    n = int(round(frac * wl.batch))
    bt = inp["block_table_host"]
    cache = inp["kv_cache"]
    done = 0
    for b in rng.choice(wl.batch, size=n, replace=False):
        b = int(b)
        s = int(rng.integers(wl.num_shards))
        lo, hi = (int(x) for x in bounds_np[b, s])
        if hi - lo < 2:
            continue
        t = (lo + hi) // 2
        h = int(rng.integers(wl.num_q_heads))
        qh = q_dev[b].reshape(-1, wl.head_dim_qk)[h].float()
        c = score / (wl.softmax_scale * float(qh @ qh))
        cache[int(bt[b, t // wl.block_size]), t % wl.block_size] = (c * qh).to(cache.dtype)
        done += 1
    torch.cuda.synchronize()
    return done


# ------------------------------------------------------------------ HBM read ceiling

def hbm_read_ceiling(dev, gib, launches=10):
    """Read rate of a plain streaming kernel (dcp_hbm_read_ceiling: 128-bit non-temporal loads
    over every CU) on a `gib` GiB buffer, timed with HIP events on the stream it runs on."""
    import torch
    import sequence_sharded_kv_amd as dcp
    n = int(gib * (1 << 30)) // 16 * 16
    buf = torch.zeros(n, dtype=torch.uint8, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    sink = torch.empty(2 * cus, dtype=torch.int32, device=dev)
    for _ in range(2):
        dcp.dcp_hbm_read_ceiling(buf, sink)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(launches):
        dcp.dcp_hbm_read_ceiling(buf, sink)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / launches
    del buf, sink
    gbs = n / (ms * 1e-3) / 1e9
    return {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes_per_launch": n, "launches": launches, "ms_per_launch": round(ms, 4),
            "kernel": "stream_read_kernel"}


# ------------------------------------------------------------------ CPU baseline

def host_info():
    """CPU model, logical CPUs visible to this process and RAM of the host."""
    model, ram = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    ram = round(int(line.split()[1]) / (1 << 20), 1)
                    break
    except OSError:
        pass
    try:
        visible = len(os.sched_getaffinity(0))
    except OSError:
        visible = os.cpu_count()
    return {"cpu_model": model, "logical_cpus_visible": visible, "ram_gib": ram}


def cpu_baseline(wl, inp, bounds_np, seconds):
    """The float64 oracle, as it stands, on whole sequences drawn in a seeded order until
    about `seconds` of CPU time; throughput in the GPU value's unit (TB/s of the step's
    algorithmic bytes, scaled to the sample)."""
    import torch
    from oracle import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    lens = inp["seq_lens_host"]
    bt = inp["block_table_host"]
    order = np.random.default_rng(7).permutation(wl.batch)
    names = ("kv_cache",) if wl.kind == "mla" else ("k_cache", "v_cache")

    def host(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    q_all = host(inp["q"])
    elapsed, done = 0.0, []
    for b in order:
        b = int(b)
        n = -(-int(lens[b]) // wl.block_size)
        idx = torch.from_numpy(bt[b, :n].astype(np.int64)).to(inp["q"].device)
        caches = tuple(host(inp[nm].index_select(0, idx)) for nm in names)
        table = np.arange(max(n, 1), dtype=np.int32)[None, :]
        t0 = time.perf_counter()
        po, pl = O.partial_attention(wl.kind, wl.dtype, q_all[b:b + 1], caches, table,
                                     bounds_np[b:b + 1].astype(np.int64), wl.block_size,
                                     wl.softmax_scale, wl.head_dim_v)
        O.merge_lse(po, pl)
        elapsed += time.perf_counter() - t0
        done.append(b)
        if elapsed >= seconds:
            break
    sample = byte_model(wl.replace(batch=len(done)), lens[done])
    return {"value": sample["step"] / elapsed / 1e12, "unit": "TB/s", "cores": int(threads),
            "kind": "oracle", **host_info(),
            "sample": f"{len(done)} of {wl.batch} requests ({sample['tokens']} tokens, all "
                      f"{wl.num_shards} shards + merge), float64 numpy, {elapsed:.1f} s"}


# ------------------------------------------------------------------ main

def time_append(wl, sh, inp, k_cache, v_cache, dev, n, busy):
    """Time dcp_append_kv storing one new row per request (after the attention timing, so the
    attention inputs are untouched while they are measured). Each request rewrites the slot
    of its last cached token, which its block table always covers. `busy` queues one
    attention step first: while the GPU runs it, the host queues all n appends, so the
    events between them time back-to-back launches rather than the host's call rate."""
    import torch
    import sequence_sharded_kv_amd as dcp
    from workloads import make_new_rows
    rows = make_new_rows(wl)
    dev_rows = {}
    for k, a in rows.items():
        t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
        dev_rows[k] = t.view(torch.bfloat16) if a.dtype == np.uint16 else t
    nk = dev_rows["new_latent"] if wl.kind == "mla" else dev_rows["new_k"]
    nv = None if wl.kind == "mla" else dev_rows["new_v"]
    pos = torch.clamp(inp["seq_lens"] - 1, min=0).to(torch.int32)
    owner = torch.empty(wl.batch, dtype=torch.int32, device=dev)

    def call():
        dcp.dcp_append_kv(sh, pos, nk, nv, inp["block_table"], k_cache, v_cache, owner)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    assert int(owner.min()) >= 0
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    busy()
    a.record()
    for _ in range(n):
        call()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    esz = 2 if wl.dtype == "bf16" else 4
    heads = 1 if wl.kind == "mla" else wl.num_kv_heads
    row = heads * (wl.head_dim_qk + (0 if wl.kind == "mla" else wl.head_dim_v)) * esz
    nbytes = wl.batch * (2 * row + 3 * 4)   # new rows read, cache rows written, len/table/owner
    return {"us_per_launch": round(us, 3), "launches": n, "algorithmic_bytes": nbytes,
            "achieved_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "bound": "launch latency (one row per request, launches queued back to back)"}


def main():
    args = parse_args()
    from workloads import make_device_inputs, workload
    wl = workload(args.workload)
    family = kernel_family(wl, args.q_len)
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc, args.workload, family,
                                       args.pmc_calibration_gib), indent=1))
        return 0
    if args.summarize_mfma:
        print(json.dumps(summarize_mfma(args.summarize_mfma, args.workload, family, wl),
                         indent=1))
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this build runs every shard on one device and issues "
              f"no collectives (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        return 2
    import torch
    import sequence_sharded_kv_amd as dcp
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    inp = make_device_inputs(wl, dev, seed=args.seed)
    lens = inp["seq_lens_host"]
    bounds_np = dcp.dcp_plan_shards(lens, wl.num_shards, wl.block_size)
    bounds = torch.from_numpy(bounds_np).to(dev)
    sh = dcp.make_shape(wl.kind, wl.dtype, wl.batch, wl.num_q_heads, wl.num_kv_heads,
                        wl.head_dim_qk, wl.head_dim_v, wl.block_size,
                        int(inp["block_table_host"].shape[1]), int(inp["num_blocks"]),
                        wl.num_shards, wl.softmax_scale)
    T = args.q_len
    ws = dcp.alloc_workspace(sh, dev, T)
    out = torch.empty((wl.batch, T, wl.num_q_heads, wl.head_dim_v), dtype=torch.float32,
                      device=dev)
    out_lse = torch.empty((wl.batch, T, wl.num_q_heads), dtype=torch.float32, device=dev)
    if T > 1:
        from workloads import make_queries
        qh = make_queries(wl, T, seed=args.seed)
        q_dev = torch.from_numpy(qh.view(np.int16) if qh.dtype == np.uint16 else qh).to(dev)
        if qh.dtype == np.uint16:
            q_dev = q_dev.view(torch.bfloat16)
    else:
        q_dev = inp["q"]
    k_cache = inp["kv_cache"] if wl.kind == "mla" else inp["k_cache"]
    v_cache = None if wl.kind == "mla" else inp["v_cache"]
    torch.cuda.synchronize()
    print(f"[bench] {wl.name}: inputs ready in {time.perf_counter() - t_gen:.1f} s, "
          f"{int(lens.sum())} tokens", file=sys.stderr, flush=True)

    def step():
        if T == 1:
            dcp.dcp_decode_attn(sh, q_dev, k_cache, v_cache, inp["block_table"], bounds, ws, out,
                                out_lse)
        else:
            dcp.dcp_decode_attn_multi(sh, T, q_dev, k_cache, v_cache, inp["block_table"], bounds,
                                      ws, out, out_lse)

    if args.calibration_copy_gib > 0:
        n = int(args.calibration_copy_gib * (1 << 30) // 4)
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b
    planted = None
    if args.plant_high_keys > 0:
        if wl.kind != "mla":
            print("--plant-high-keys applies to MLA workloads", file=sys.stderr)
            return 2
        n = plant_high_keys(wl, inp, bounds_np, q_dev, args.plant_high_keys)
        planted = {"requests": n, "score_nats": 90.0}
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    flags = dcp.dcp_read_device_flags(ws)
    # bits 0 and 1 are input errors; bits 2 and 3 are informational (a worker recomputed its
    # range, or raised a row's reference and rescaled it in place) and are reported
    assert flags & 3 == 0, flags
    if planted is not None:
        planted["device_flags"] = flags
    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    dcp.dcp_kernel_timing_begin(2 * K)  # room for two passes per step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        starts[i].record()
        step()
        ends[i].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launches, kernel_ms = dcp.dcp_kernel_timing_end()
    per_step = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    ms_per_step = (t1 - t0) * 1e3 / K
    bm = byte_model(wl, lens, T)
    value = bm["step"] / (ms_per_step * 1e-3) / 1e12
    # per step: a fused call that runs its query tokens in two passes times two launches
    kern_avg_ms = kernel_ms / K
    achieved = bm["partial_kernel"] / (kern_avg_ms * 1e-3) / 1e9
    traffic = load_traffic(wl.name, family) if T == 1 else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else int(traffic["traffic_bytes_per_launch"]),
                "kernel": KERNEL_NAMES[family], "kernel_avg_ms": round(kern_avg_ms, 4),
                "launches_per_step": round(launches / K, 3),
                "algorithmic_bytes_per_launch": int(bm["partial_kernel"])}
    # matrix-unit use of the same kernel, from a committed rocprofv3 --pmc summary taken on
    # the same kernel sources (null once they have changed)
    mf = load_traffic(wl.name, family, mfma_file(wl.name)) if T == 1 else None
    mfma = None
    if mf is not None:
        issued = mf["mfma_flops_per_launch"] / (kern_avg_ms * 1e-3) / 1e12
        algo = flop_model(wl, lens, 1)
        mfma = {"busy_pct": round(mf["mfma_busy_pct"], 2),
                "issued_tflops": round(issued, 1), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                "issued_frac": round(issued / MFMA_BF16_PEAK_TFLOPS, 4),
                "issued_flops_per_launch": int(mf["mfma_flops_per_launch"]),
                "algorithmic_flops_per_launch": int(algo)}
    prefill = T > 16   # a prefill chunk: compute-bound, measured in flops
    if prefill:
        flops = flop_model(wl, lens, T)
        value = flops / (ms_per_step * 1e-3) / 1e12
        achieved = flops / (kern_avg_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": KERNEL_NAMES[family], "kernel_avg_ms": round(kern_avg_ms, 4),
                    "algorithmic_flops_per_launch": int(flops)}
    append = time_append(wl, sh, inp, k_cache, v_cache, dev, 200, step)
    ceiling = None
    if args.ceiling_gib > 0:
        ceiling = hbm_read_ceiling(dev, args.ceiling_gib)
        if roofline["unit"] == "GB/s":
            roofline["frac_of_read_ceiling"] = round(roofline["achieved"] / ceiling["GBps"], 4)
    cpu = None
    if not args.no_cpu_baseline and T == 1:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, bounds_np, args.cpu_seconds)
    q = np.percentile(per_step, [10, 50, 90])
    if prefill:
        metric, unit = (f"sharded chunked-prefill attention algorithmic TFLOP/s ({T}-token causal "
                        "chunk against the sharded cache)"), "TFLOP/s"
    elif wl.kind == "mla":
        metric, unit = ("sharded decode-attn achieved HBM TB/s (% peak) + decode steps/s, MLA 67K "
                        "ctx"), "TB/s"
    else:
        metric, unit = "sharded decode-attn achieved HBM TB/s (% peak) + decode steps/s", "TB/s"
    line = {
        "metric": metric,
        "value": round(value, 4), "unit": unit, "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "steps_per_s": round(1e3 / ms_per_step, 2),
        "pct_of_hbm_peak": None if prefill else round(100 * value * 1e3 / HBM_PEAK_GBS, 2),
        "ms_per_step_p10_p50_p90": [round(float(x), 4) for x in q],
        "config": {"workload": wl.name if T == 1 else f"{wl.name}-q{T}", "kind": wl.kind,
                   "batch": wl.batch, "query_tokens": T,
                   "num_q_heads": wl.num_q_heads, "num_kv_heads": wl.num_kv_heads,
                   "head_dim_qk": wl.head_dim_qk, "head_dim_v": wl.head_dim_v,
                   "block_size": wl.block_size, "num_shards": wl.num_shards,
                   "tokens": bm["tokens"], "context_median": int(np.median(lens)),
                   "kv_bytes": bm["kv"], "algorithmic_bytes_per_step": bm["step"],
                   "parallelism": "all shards on one GPU"},
        "roofline": roofline,
        "mfma": mfma,
        "hbm_read_ceiling": ceiling,
        "planted_high_keys": planted,
        "device_flags": flags,
        "cpu_baseline": cpu,
        "append_kv": append,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
