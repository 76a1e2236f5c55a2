"""Host-side logic of bench.py: the byte and flop models, the kernel-family choice, the two
rocprofv3 counter summaries and the one-GPU refusal. No GPU is touched."""

import csv
import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from workloads import workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_byte_model_counts_each_stream_once(bench):
    # MLA: the value is the first 512 of the 576 cached dims, so the KV is 576 bf16 per token
    wl = workload("mla-64h-b512").replace(batch=2)
    lens = np.array([100, 64], np.int64)
    bm = bench.byte_model(wl, lens, 1)
    assert bm["kv"] == 164 * 576 * 2
    assert bm["q"] == 2 * 64 * 576 * 2
    assert bm["table"] == (2 + 1) * 4                      # ceil(100/64) + ceil(64/64) pages
    part = 2 * 8 * 64 * (512 + 1) * 4
    assert bm["partials_rw"] == 2 * part
    assert bm["out"] == 2 * 64 * 513 * 4
    assert bm["step"] == bm["kv"] + bm["q"] + bm["table"] + 2 * part + bm["out"]
    assert bm["partial_kernel"] == bm["kv"] + bm["q"] + bm["table"] + part
    # GQA: K and V, one row per KV head; several query tokens do not add KV bytes
    g = workload("gqa-g16").replace(batch=1)
    b1 = bench.byte_model(g, np.array([33]), 1)
    b3 = bench.byte_model(g, np.array([33]), 3)
    assert b1["kv"] == 33 * 4 * 128 * 2 * 2 == b3["kv"]
    assert b3["q"] == 3 * b1["q"]


def test_flop_model_is_the_causal_sum(bench):
    wl = workload("mla-64h-b512").replace(batch=2)
    lens = np.array([5, 9])
    per = 2 * 576 + 2 * 512
    assert bench.flop_model(wl, lens, 1) == (5 + 9) * 64 * per
    # query j of T sees L - T + j + 1 positions
    vis = sum(max(0, L - 3 + j + 1) for L in (5, 9) for j in range(3))
    assert bench.flop_model(wl, lens, 3) == vis * 64 * per
    assert bench.flop_model(wl, np.array([2]), 4) == (0 + 0 + 1 + 2) * 64 * per


def test_kernel_family_follows_the_row_count(bench):
    assert bench.kernel_family(workload("mla-64h-b512"), 1) == "mla-ring"   # 64 rows, 12 waves
    assert bench.kernel_family(workload("mla-64h-b512").replace(num_q_heads=32), 1) == "mla"
    assert bench.kernel_family(workload("mla-64h-b512").replace(num_q_heads=32), 2) == "mla-ring"
    assert bench.kernel_family(workload("mla-64h-b512").replace(num_q_heads=16), 3) == "mla-ring"
    assert bench.kernel_family(workload("mla-64h-b512").replace(num_q_heads=32), 5) == "mla-split"
    assert bench.kernel_family(workload("mla-64h-b512").replace(num_q_heads=16), 12) == "mla-split"
    assert bench.kernel_family(workload("mla-64h-b512"), 2) == "mla-pair"   # 128 rows, 8 waves
    assert bench.kernel_family(workload("mla-64h-b512"), 3) == "mla-split"   # 128 + 64 rows
    assert bench.kernel_family(workload("mla-64h-b512"), 4) == "mla-pair"   # 2 x 128 rows
    assert bench.kernel_family(workload("mla-128h"), 1) == "mla-pair"
    assert bench.kernel_family(workload("mla-64h-b512").replace(num_q_heads=16), 5) == "mla-pair"
    assert bench.kernel_family(workload("gqa-g16"), 1) == "gqa-chunk"   # 16 of 32 rows
    assert bench.kernel_family(workload("gqa-g16"), 2) == "gqa-chunk"
    assert bench.kernel_family(workload("gqa-long"), 1) == "gqa-chunk"  # 8 of 32 rows
    assert bench.kernel_family(workload("gqa-g16").replace(num_q_heads=16, head_dim_qk=64,
                                                           head_dim_v=64), 1) == "gqa-mfma"
    assert bench.kernel_family(workload("gqa-tiny"), 1) == "gqa-valu"   # fp32


def _write_counters(path, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_traffic_summary_scales_by_the_reference_pass(bench, tmp_path):
    fam = "gqa-mfma"
    kname = bench.KERNEL_NAMES[fam]
    fd, wd = tmp_path / "f", tmp_path / "w"
    fd.mkdir()
    wd.mkdir()
    gib_kib = 1 << 20
    # the counter reads half the true bytes for the 1 GiB pass: scale 2
    _write_counters(fd / "run_counter_collection.csv", [
        (0, "distribution_elementwise_grid_stride_kernel<float>", "FETCH_SIZE", 3 * gib_kib),
        (1, "elementwise_kernel<float>", "FETCH_SIZE", gib_kib / 2),
        (2, f"void dcp::{kname}<128>(...)", "FETCH_SIZE", 1000.0),
        (3, f"void dcp::{kname}<128>(...)", "FETCH_SIZE", 3000.0),
        (4, "void dcp::merge_kernel(...)", "FETCH_SIZE", 99999.0)])
    _write_counters(wd / "run_counter_collection.csv", [
        (0, "distribution_elementwise_grid_stride_kernel<float>", "WRITE_SIZE", gib_kib / 2),
        (1, "elementwise_kernel<float>", "WRITE_SIZE", gib_kib),
        (2, f"void dcp::{kname}<128>(...)", "WRITE_SIZE", 10.0),
        (5, "elementwise_kernel<float>", "WRITE_SIZE", 7 * gib_kib)])
    t = bench.summarize_pmc(str(fd), str(wd), "gqa-g16", fam, 1.0)
    assert t["fetch_size_calibration_scale"] == pytest.approx(2.0)
    assert t["write_size_calibration_scale"] == pytest.approx(1.0)
    assert t["fetch_size_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2)
    assert t["write_size_bytes_per_launch"] == pytest.approx(10.0 * 1024)
    assert t["fetch_size_dispatches"] == 2
    assert t["traffic_bytes_per_launch"] == pytest.approx(2000.0 * 2048 + 10240)
    assert t["kernel_sources_sha256"] == bench.sources_sha(fam)
    # without a reference pass of about the stated size before the kernel there is no scale
    _write_counters(wd / "run_counter_collection.csv", [
        (1, "elementwise_kernel<float>", "WRITE_SIZE", gib_kib / 64),
        (2, f"void dcp::{kname}<128>(...)", "WRITE_SIZE", 10.0)])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(fd), str(wd), "gqa-g16", fam, 1.0)


def test_mfma_summary_averages_the_kernel_dispatches(bench, tmp_path):
    fam = "mla"
    kname = bench.KERNEL_NAMES[fam]
    _write_counters(tmp_path / "run_counter_collection.csv", [
        (1, "void dcp::schedule_kernel(...)", "MfmaUtil", 0.0),
        (2, f"void dcp::{kname}<4>(...)", "MfmaUtil", 30.0),
        (3, f"void dcp::{kname}<4>(...)", "MfmaUtil", 40.0),
        (2, f"void dcp::{kname}<4>(...)", "MfmaFlopsBF16", 16384.0 * 10),
        (3, f"void dcp::{kname}<4>(...)", "MfmaFlopsBF16", 16384.0 * 30),
        (2, f"void dcp::{kname}<4>(...)", "SQ_INSTS_VALU_MFMA_BF16", 10.0),
        (3, f"void dcp::{kname}<4>(...)", "SQ_INSTS_VALU_MFMA_BF16", 30.0)])
    m = bench.summarize_mfma(str(tmp_path), "mla-64h-b512", fam, workload("mla-64h-b512"))
    assert m["mfma_busy_pct"] == pytest.approx(35.0)
    assert m["mfma_flops_per_launch"] == pytest.approx(16384.0 * 20)
    assert m["flops_per_instruction"] == pytest.approx(16384.0)
    assert m["mfma_busy_pct_dispatches"] == 2


def test_counter_files_are_ignored_once_the_kernel_changes(bench, tmp_path):
    p = tmp_path / "t.json"
    p.write_text(json.dumps({"kernel_sources_sha256": "0" * 64, "traffic_bytes_per_launch": 1}))
    assert bench.load_traffic("gqa-g16", "gqa-mfma", str(p)) is None
    p.write_text(json.dumps({"kernel_sources_sha256": bench.sources_sha("gqa-mfma"),
                             "traffic_bytes_per_launch": 1}))
    assert bench.load_traffic("gqa-g16", "gqa-mfma", str(p))["traffic_bytes_per_launch"] == 1


def test_committed_counter_files_name_their_kernel(bench):
    prof = os.path.join(ROOT, "profiles")
    for f in sorted(os.listdir(prof)):
        if f.endswith(".json") and (f.startswith("traffic_") or f.startswith("mfma_")):
            t = json.load(open(os.path.join(prof, f)))
            wl = workload(t["workload"])
            assert t["kernel"] == bench.KERNEL_NAMES[bench.kernel_family(wl, 1)], f
            assert len(t["kernel_sources_sha256"]) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
