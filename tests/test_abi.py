"""The C ABI without a GPU: exports, version, status strings, host plan and every
host-checked error path (each must return before any HIP call)."""

import ctypes
import os
import re

import numpy as np
import pytest

import sequence_sharded_kv_amd as dcp
from oracle import plan_shards as oracle_plan

def _gpu_visible():
    """Counting devices does not initialise the GPU."""
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001
        return False


# These tests pass fabricated device addresses into entry points that launch kernels once
# validation passes; every call is built to fail validation first. On a host with a GPU a
# reordered check could launch on a bogus address, so they run only where no GPU is visible.
fake_addresses = pytest.mark.skipif(
    _gpu_visible(), reason="fabricated device addresses: run on a host without a GPU")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "dcp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcp_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = dcp.load()
    # DCP_LIBRARY selects another build of the library (the sanitized one)
    assert lib._name == (os.environ.get("DCP_LIBRARY") or dcp.LIB_PATH)
    names = declared_functions()
    assert len(names) == 19, names
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(dcp.EXPORTS) == names


def test_version_and_status_strings():
    assert dcp.dcp_abi_version() == 1
    for s in range(8):
        assert dcp.dcp_status_string(s)
    assert dcp.dcp_status_string(99) == "unknown status"


def test_host_plan_matches_oracle_bit_exact():
    rng = np.random.default_rng(0)
    for _ in range(200):
        B = int(rng.integers(1, 9))
        S = int(rng.integers(1, 33))
        bs = int(rng.choice([1, 16, 64]))
        lens = rng.integers(0, 300_000, size=B).astype(np.int32)
        lens[rng.random(B) < 0.2] = rng.integers(0, 3)
        got = dcp.dcp_plan_shards(lens, S, bs)
        want = oracle_plan(lens.tolist(), S, bs)
        assert got.dtype == np.int32 and np.array_equal(got.astype(np.int64), want)


def test_host_plan_pages_example():
    got = dcp.dcp_plan_shards([200_000, 1_000_000], 4, 16)
    assert got[0].tolist() == [[0, 50_000], [50_000, 100_000], [100_000, 150_000],
                               [150_000, 200_000]]
    got = dcp.dcp_plan_shards([1_000_000], 16, 16)
    assert got[0, -1].tolist() == [937_680, 1_000_000]
    assert (got[0, :, 1] - got[0, :, 0]).tolist() == [62_512] * 15 + [62_320]


@pytest.mark.parametrize("args,code", [
    (([5], 0, 16), dcp.DCP_ERR_SHAPE),
    (([5], 4, 0), dcp.DCP_ERR_SHAPE),
    (([5, -1], 4, 16), dcp.DCP_ERR_BAD_PLAN),
])
def test_host_plan_errors(args, code):
    with pytest.raises(dcp.DcpError) as e:
        dcp.dcp_plan_shards(*args)
    assert e.value.status == code


def _shape(**kw):
    base = dict(kind="mla", dtype="bf16", batch=4, num_q_heads=64, num_kv_heads=1, head_dim_qk=576,
                head_dim_v=512, block_size=64, max_blocks_per_seq=16, num_blocks=64, num_shards=8,
                softmax_scale=192 ** -0.5)
    base.update(kw)
    return dcp.make_shape(**base)


def test_workspace_bytes_and_shape_errors():
    n = dcp.dcp_workspace_bytes(_shape())
    assert n > 4 * 8 * 64 * 512 * 4
    assert n % 256 == 0
    bad = [
        dict(batch=0), dict(num_shards=0), dict(block_size=0), dict(num_q_heads=60, num_kv_heads=8),
        dict(kind="gqa", head_dim_v=64), dict(num_kv_heads=2, num_q_heads=64),
        dict(dtype="fp8"), dict(kind="xyz"), dict(softmax_scale=float("inf")),
        dict(head_dim_v=510, head_dim_qk=576),
    ]
    for kw in bad:
        with pytest.raises(dcp.DcpError) as e:
            dcp.dcp_workspace_bytes(_shape(**kw))
        assert e.value.status == dcp.DCP_ERR_SHAPE, kw
    unsupported = [dict(num_q_heads=48), dict(dtype="f32"), dict(head_dim_qk=320, head_dim_v=256),
                   dict(kind="gqa", num_q_heads=64, num_kv_heads=2, head_dim_qk=128,
                        head_dim_v=128)]
    for kw in unsupported:
        with pytest.raises(dcp.DcpError) as e:
            dcp.dcp_workspace_bytes(_shape(**kw))
        assert e.value.status == dcp.DCP_ERR_UNSUPPORTED, kw


class _Fake:
    """Stands in for a device tensor: only its address is used before validation fails."""

    def __init__(self, addr, nbytes=1 << 20):
        self.addr, self.nbytes = addr, nbytes

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


def _call_partial(sh, q, k, v, bt, bounds, po, pl, ws):
    lib = dcp.load()
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return lib.dcp_decode_attn_partial(ctypes.byref(sh), p(q), p(k), p(v), p(bt), p(bounds),
                                       p(po), p(pl), p(ws), ws.nbytes if ws else 0, None)


@fake_addresses
def test_partial_error_paths_return_before_device_work():
    sh = _shape()
    need = dcp.dcp_workspace_bytes(sh)
    A = lambda: _Fake(0x10000)  # noqa: E731
    ws_ok = _Fake(0x20000, need)
    assert _call_partial(sh, None, A(), None, A(), A(), A(), A(), ws_ok) == dcp.DCP_ERR_NULL
    assert _call_partial(sh, A(), A(), A(), A(), A(), A(), A(), ws_ok) == dcp.DCP_ERR_SHAPE
    assert _call_partial(sh, _Fake(0x10008), A(), None, A(), A(), A(), A(), ws_ok) == \
        dcp.DCP_ERR_ALIGN
    assert _call_partial(sh, A(), A(), None, A(), A(), A(), A(), _Fake(0x20000, need - 1)) == \
        dcp.DCP_ERR_WORKSPACE
    gqa = _shape(kind="gqa", num_q_heads=8, num_kv_heads=2, head_dim_qk=64, head_dim_v=64)
    assert _call_partial(gqa, A(), A(), None, A(), A(), A(), A(), ws_ok) == dcp.DCP_ERR_NULL
    assert "v_cache" in dcp.dcp_last_error()


@fake_addresses
def test_merge_and_fused_error_paths():
    lib = dcp.load()
    assert lib.dcp_merge_lse(2, 4, 8, 64, None, 0x1000, 0x2000, None, None) == dcp.DCP_ERR_NULL
    assert lib.dcp_merge_lse(2, 4, 8, 62, 0x1000, 0x1000, 0x2000, None, None) == dcp.DCP_ERR_SHAPE
    assert lib.dcp_merge_lse(0, 4, 8, 64, 0x1000, 0x1000, 0x2000, None, None) == dcp.DCP_ERR_SHAPE
    assert lib.dcp_merge_lse(2, 4, 8, 64, 0x1004, 0x1000, 0x2000, None, None) == dcp.DCP_ERR_ALIGN
    sh = _shape()
    assert lib.dcp_decode_attn(ctypes.byref(sh), 0x1000, 0x1000, None, 0x1000, 0x1000, 0x1000, 16,
                               None, None, None) == dcp.DCP_ERR_NULL
    assert lib.dcp_decode_attn(ctypes.byref(sh), 0x1000, 0x1000, None, 0x1000, 0x1000, 0x1000, 16,
                               0x3000, None, None) == dcp.DCP_ERR_WORKSPACE
    assert lib.dcp_debug_gather_shard(ctypes.byref(sh), 0x1000, 0x1000, 0x1000, 9, 0, 0, 0x1000, 4,
                                      None) == dcp.DCP_ERR_SHAPE
    assert lib.dcp_read_device_flags(None, None, None) == dcp.DCP_ERR_NULL
    assert lib.dcp_kernel_timing_begin(0) == dcp.DCP_ERR_SHAPE
    assert lib.dcp_kernel_timing_end(None, None) == dcp.DCP_ERR_NULL


@fake_addresses
def test_noalloc_limit_and_error_paths_return_before_device_work():
    """The no-allocation entry point states its scratch size in the header and refuses a
    shape whose workspace exceeds it before touching the device."""
    text = open(HEADER).read()
    m = re.search(r"#define DCP_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == dcp.DCP_NOALLOC_SCRATCH_BYTES
    lib = dcp.load()
    A = 0x10000
    big = _shape(batch=512, num_shards=8)  # 64 heads x 512 dims x 4096 shards of partials
    assert dcp.dcp_workspace_bytes(big) > dcp.DCP_NOALLOC_SCRATCH_BYTES
    assert lib.dcp_decode_attn_noalloc(ctypes.byref(big), A, A, None, A, A, A, None, None) == \
        dcp.DCP_ERR_WORKSPACE
    assert "static scratch" in dcp.dcp_last_error()
    small = _shape()
    assert dcp.dcp_workspace_bytes(small) <= dcp.DCP_NOALLOC_SCRATCH_BYTES
    assert lib.dcp_decode_attn_noalloc(ctypes.byref(small), None, A, None, A, A, A, None,
                                       None) == dcp.DCP_ERR_NULL
    assert lib.dcp_decode_attn_noalloc(ctypes.byref(small), A, A, None, A, A, None, None,
                                       None) == dcp.DCP_ERR_NULL
    assert lib.dcp_decode_attn_noalloc(None, A, A, None, A, A, A, None, None) == dcp.DCP_ERR_NULL
    bad = _shape(num_shards=0)
    assert lib.dcp_decode_attn_noalloc(ctypes.byref(bad), A, A, None, A, A, A, None, None) == \
        dcp.DCP_ERR_SHAPE


@fake_addresses
def test_append_error_paths_return_before_device_work():
    lib = dcp.load()
    A = 0x10000

    def call(sh, lens=A, nk=A, nv=None, bt=A, kc=A, vc=None, owner=None):
        return lib.dcp_append_kv(ctypes.byref(sh), lens, nk, nv, bt, kc, vc, owner, None)

    mla = _shape()
    assert call(mla, lens=None) == dcp.DCP_ERR_NULL
    assert call(mla, nk=None) == dcp.DCP_ERR_NULL
    assert call(mla, bt=None) == dcp.DCP_ERR_NULL
    assert call(mla, kc=None) == dcp.DCP_ERR_NULL
    assert call(mla, nv=A) == dcp.DCP_ERR_SHAPE
    assert call(mla, vc=A) == dcp.DCP_ERR_SHAPE
    assert call(mla, nk=A + 8) == dcp.DCP_ERR_ALIGN
    assert call(mla, kc=A + 2) == dcp.DCP_ERR_ALIGN
    assert call(_shape(batch=0)) == dcp.DCP_ERR_SHAPE
    # 36 bf16 dims = 72 bytes: not whole 16-byte chunks
    assert call(_shape(head_dim_qk=36, head_dim_v=32)) == dcp.DCP_ERR_UNSUPPORTED
    gqa = _shape(kind="gqa", num_q_heads=8, num_kv_heads=2, head_dim_qk=64, head_dim_v=64)
    assert call(gqa) == dcp.DCP_ERR_NULL
    assert "new_v" in dcp.dcp_last_error()
    assert call(gqa, nv=A) == dcp.DCP_ERR_NULL
    assert call(gqa, nv=A + 4, vc=A) == dcp.DCP_ERR_ALIGN
    gqa_odd = _shape(kind="gqa", num_q_heads=8, num_kv_heads=2, head_dim_qk=4, head_dim_v=4)
    assert call(gqa_odd, nv=A, vc=A) == dcp.DCP_ERR_UNSUPPORTED


@fake_addresses
def test_multi_token_shapes_and_errors():
    sh = _shape()
    one = dcp.dcp_workspace_bytes(sh)
    assert dcp.dcp_workspace_bytes_multi(sh, 1) == one
    assert dcp.dcp_workspace_bytes_multi(sh, 4) > one
    assert dcp.dcp_workspace_bytes_multi(sh, 4096) > dcp.dcp_workspace_bytes_multi(sh, 16)
    for bad in (0, 4097, -1):
        with pytest.raises(dcp.DcpError) as e:
            dcp.dcp_workspace_bytes_multi(sh, bad)
        assert e.value.status == dcp.DCP_ERR_SHAPE
    lib = dcp.load()
    A = 0x10000
    need = dcp.dcp_workspace_bytes_multi(sh, 3)
    assert lib.dcp_decode_attn_multi(ctypes.byref(sh), 3, A, A, None, A, A, A, need - 1, A, None,
                                     None) == dcp.DCP_ERR_WORKSPACE
    assert lib.dcp_decode_attn_multi(ctypes.byref(sh), 0, A, A, None, A, A, A, need, A, None,
                                     None) == dcp.DCP_ERR_SHAPE
    assert lib.dcp_decode_attn_multi_partial(ctypes.byref(sh), 2, A, A, None, A, A, None, A, A,
                                             need, None) == dcp.DCP_ERR_NULL
    # a two-pass call (64 heads x 3 tokens) checks the workspace before its first launch
    assert lib.dcp_decode_attn_multi_partial(ctypes.byref(sh), 3, A, A, None, A, A, A, A, A,
                                             need - 1, None) == dcp.DCP_ERR_WORKSPACE


def test_workspace_of_a_two_pass_call_holds_each_pass():
    """MLA calls of 129 to 192 query rows run a 128-row pass (128 / Hq tokens) and a pass
    with the remaining tokens in the same workspace: the size reported for the call covers
    the single-pass plans of both token counts."""
    for hq, q_len in ((64, 3), (32, 5), (32, 6), (16, 9), (16, 12)):
        sh = _shape(num_q_heads=hq)
        ta = 128 // hq
        need = dcp.dcp_workspace_bytes_multi(sh, q_len)
        assert need >= dcp.dcp_workspace_bytes_multi(sh, ta)
        assert need >= dcp.dcp_workspace_bytes_multi(sh, q_len - ta)
    # 64 heads x 3 tokens: the 128-row pass keeps pieces of 128 rows per worker, more than
    # the partial call's three 64-row units need
    sh = _shape(num_q_heads=64)
    assert dcp.dcp_workspace_bytes_multi(sh, 3) == dcp.dcp_workspace_bytes_multi(sh, 2)
