"""ctypes binding of libdcp.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/dcp.h); all the
work of the path runs in the library's HIP kernels. Device arguments are torch tensors on
a ROCm device; the call is queued on torch's current stream of that device.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdcp.so")

DCP_OK = 0
DCP_ERR_NULL = 1
DCP_ERR_SHAPE = 2
DCP_ERR_UNSUPPORTED = 3
DCP_ERR_WORKSPACE = 4
DCP_ERR_BAD_PLAN = 5
DCP_ERR_ALIGN = 6
DCP_ERR_DEVICE = 7

DCP_F32 = 0
DCP_BF16 = 1
DCP_KV_GQA = 0
DCP_KV_MLA = 1

EXPORTS = (
    "dcp_abi_version", "dcp_status_string", "dcp_last_error", "dcp_plan_shards",
    "dcp_plan_shards_device", "dcp_workspace_bytes", "dcp_decode_attn_partial", "dcp_merge_lse",
    "dcp_decode_attn", "dcp_read_device_flags", "dcp_debug_gather_shard",
    "dcp_kernel_timing_begin", "dcp_kernel_timing_end", "dcp_append_kv",
    "dcp_workspace_bytes_multi", "dcp_decode_attn_multi_partial", "dcp_decode_attn_multi",
    "dcp_decode_attn_noalloc", "dcp_hbm_read_ceiling",
)

# device scratch of dcp_decode_attn_noalloc (DCP_NOALLOC_SCRATCH_BYTES)
DCP_NOALLOC_SCRATCH_BYTES = 256 << 20


class DcpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"dcp status {status}: {detail}")
        self.status = status
        self.detail = detail


class dcp_attn_shape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim_qk", ctypes.c_int32),
        ("head_dim_v", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
        ("num_shards", ctypes.c_int32), ("dtype", ctypes.c_int32), ("kv_kind", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


_lib: Optional[ctypes.CDLL] = None


def load(path: str = None) -> ctypes.CDLL:
    """Load libdcp.so (built in-tree); raises if it has not been built. DCP_LIBRARY in the
    environment names another build of the same library (the host-sanitized one of the CPU
    ABI tests)."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("DCP_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sequence_sharded_kv_amd._build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SH = ctypes.POINTER(dcp_attn_shape)
    sig = {
        "dcp_abi_version": (I32, []),
        "dcp_status_string": (ctypes.c_char_p, [I32]),
        "dcp_last_error": (ctypes.c_char_p, []),
        "dcp_plan_shards": (I32, [P, I32, I32, I32, P]),
        "dcp_plan_shards_device": (I32, [P, I32, I32, I32, P, P]),
        "dcp_workspace_bytes": (I32, [SH, ctypes.POINTER(SZ)]),
        "dcp_decode_attn_partial": (I32, [SH, P, P, P, P, P, P, P, P, SZ, P]),
        "dcp_merge_lse": (I32, [I32, I32, I32, I32, P, P, P, P, P]),
        "dcp_decode_attn": (I32, [SH, P, P, P, P, P, P, SZ, P, P, P]),
        "dcp_read_device_flags": (I32, [P, ctypes.POINTER(I32), P]),
        "dcp_debug_gather_shard": (I32, [SH, P, P, P, I32, I32, I32, P, I32, P]),
        "dcp_kernel_timing_begin": (I32, [I32]),
        "dcp_kernel_timing_end": (I32, [ctypes.POINTER(I32), ctypes.POINTER(ctypes.c_float)]),
        "dcp_append_kv": (I32, [SH, P, P, P, P, P, P, P, P]),
        "dcp_workspace_bytes_multi": (I32, [SH, I32, ctypes.POINTER(SZ)]),
        "dcp_decode_attn_multi_partial": (I32, [SH, I32, P, P, P, P, P, P, P, P, SZ, P]),
        "dcp_decode_attn_multi": (I32, [SH, I32, P, P, P, P, P, P, SZ, P, P, P]),
        "dcp_decode_attn_noalloc": (I32, [SH, P, P, P, P, P, P, P, P]),
        "dcp_hbm_read_ceiling": (I32, [P, SZ, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != DCP_OK:
        detail = load().dcp_last_error().decode()
        raise DcpError(status, detail or load().dcp_status_string(status).decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ------------------------------------------------------------------ argument checks
# The kernels trust the sizes in dcp_attn_shape; a tensor smaller than they say would be read
# or written out of bounds. These checks compare every tensor with the shape before the call.

def _tensor(name, t, dtype, device=None, numel=None, min_numel=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, q on {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {min_numel}")


def _elem(shape):
    import torch
    return {DCP_BF16: torch.bfloat16, DCP_F32: torch.float32}.get(shape.dtype)


def _check_attn(shape, q_len, q, k_cache, v_cache, block_table, bounds):
    """q, caches, block table and bounds against the shape (the library checks the rest)."""
    import torch
    el = _elem(shape)
    B, H = shape.batch, shape.num_q_heads
    _tensor("q", q, el, numel=B * q_len * H * shape.head_dim_qk)
    dev = q.device
    mla = shape.kv_kind == DCP_KV_MLA
    heads = 1 if mla else shape.num_kv_heads
    page_k = heads * shape.block_size * shape.head_dim_qk
    _tensor("k_cache", k_cache, el, dev, min_numel=shape.num_blocks * page_k)
    if k_cache.dim() > 1 and k_cache.shape[0] < shape.num_blocks:
        raise ValueError(f"k_cache holds {k_cache.shape[0]} pages, the shape says "
                         f"{shape.num_blocks}")
    if v_cache is not None:
        page_v = heads * shape.block_size * shape.head_dim_v
        _tensor("v_cache", v_cache, el, dev, min_numel=shape.num_blocks * page_v)
    _tensor("block_table", block_table, torch.int32, dev,
            numel=B * shape.max_blocks_per_seq)
    _tensor("bounds", bounds, torch.int32, dev, numel=B * shape.num_shards * 2)


def _check_out(shape, q_len, dev, **tensors):
    """Partials and outputs: float32 with the sizes the shape gives."""
    import torch
    B, S, H, Dv = shape.batch, shape.num_shards, shape.num_q_heads, shape.head_dim_v
    sizes = {"part_o": B * S * q_len * H * Dv, "part_lse": B * S * q_len * H,
             "out": B * q_len * H * Dv, "out_lse": B * q_len * H}
    for name, t in tensors.items():
        if t is not None:
            _tensor(name, t, torch.float32, dev, numel=sizes[name])


def _check_workspace(ws, dev):
    _tensor("workspace", ws, None, dev)


def _stream(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def make_shape(kind: str, dtype: str, batch: int, num_q_heads: int, num_kv_heads: int,
               head_dim_qk: int, head_dim_v: int, block_size: int, max_blocks_per_seq: int,
               num_blocks: int, num_shards: int, softmax_scale: float) -> dcp_attn_shape:
    return dcp_attn_shape(
        batch, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, block_size,
        max_blocks_per_seq, num_blocks, num_shards,
        DCP_BF16 if dtype == "bf16" else DCP_F32 if dtype == "f32" else -1,
        DCP_KV_MLA if kind == "mla" else DCP_KV_GQA if kind == "gqa" else -1,
        float(softmax_scale))


# ------------------------------------------------------------------ entry points

def dcp_abi_version() -> int:
    return load().dcp_abi_version()


def dcp_status_string(status: int) -> str:
    return load().dcp_status_string(status).decode()


def dcp_last_error() -> str:
    return load().dcp_last_error().decode()


def dcp_plan_shards(seq_lens, num_shards: int, block_size: int) -> np.ndarray:
    """Host plan: int32 [B, S, 2] of (start, end)."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    B = int(lens.shape[0])
    out = np.zeros((max(B, 1), num_shards if num_shards > 0 else 1, 2), dtype=np.int32)
    _check(load().dcp_plan_shards(lens.ctypes.data if B else None, B, num_shards, block_size,
                                  out.ctypes.data))
    return out


def dcp_plan_shards_device(seq_lens, num_shards: int, block_size: int, bounds=None):
    """Device plan from device int32 seq_lens into device int32 bounds [B, S, 2]."""
    import torch
    B = int(seq_lens.shape[0])
    if bounds is None:
        bounds = torch.empty((B, num_shards, 2), dtype=torch.int32, device=seq_lens.device)
    _check(load().dcp_plan_shards_device(_ptr(seq_lens), B, num_shards, block_size, _ptr(bounds),
                                         _stream(seq_lens)))
    return bounds


def dcp_workspace_bytes(shape: dcp_attn_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dcp_workspace_bytes(ctypes.byref(shape), ctypes.byref(n)))
    return int(n.value)


def dcp_decode_attn_partial(shape: dcp_attn_shape, q, k_cache, v_cache, block_table, bounds,
                            part_o, part_lse, workspace) -> None:
    _check_attn(shape, 1, q, k_cache, v_cache, block_table, bounds)
    _check_out(shape, 1, q.device, part_o=part_o, part_lse=part_lse)
    _check_workspace(workspace, q.device)
    _check(load().dcp_decode_attn_partial(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(bounds), _ptr(part_o), _ptr(part_lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))


def dcp_merge_lse(part_o, part_lse, out, out_lse=None) -> None:
    import torch
    if part_o.dim() != 4:
        raise ValueError(f"part_o must be [B][S][H][Dv], got shape {tuple(part_o.shape)}")
    B, S, H, Dv = (int(x) for x in part_o.shape)
    dev = part_o.device
    _tensor("part_o", part_o, torch.float32, dev)
    _tensor("part_lse", part_lse, torch.float32, dev, numel=B * S * H)
    _tensor("out", out, torch.float32, dev, numel=B * H * Dv)
    if out_lse is not None:
        _tensor("out_lse", out_lse, torch.float32, dev, numel=B * H)
    _check(load().dcp_merge_lse(B, S, H, Dv, _ptr(part_o), _ptr(part_lse), _ptr(out),
                                _ptr(out_lse), _stream(part_o)))


def dcp_decode_attn(shape: dcp_attn_shape, q, k_cache, v_cache, block_table, bounds, workspace,
                    out, out_lse=None) -> None:
    _check_attn(shape, 1, q, k_cache, v_cache, block_table, bounds)
    _check_out(shape, 1, q.device, out=out, out_lse=out_lse)
    _check_workspace(workspace, q.device)
    _check(load().dcp_decode_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(bounds), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _ptr(out_lse), _stream(q)))


def dcp_decode_attn_noalloc(shape: dcp_attn_shape, q, k_cache, v_cache, block_table, bounds,
                            out, out_lse=None) -> None:
    _check_attn(shape, 1, q, k_cache, v_cache, block_table, bounds)
    _check_out(shape, 1, q.device, out=out, out_lse=out_lse)
    _check(load().dcp_decode_attn_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(bounds), _ptr(out), _ptr(out_lse), _stream(q)))


def dcp_workspace_bytes_multi(shape: dcp_attn_shape, q_len: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dcp_workspace_bytes_multi(ctypes.byref(shape), q_len, ctypes.byref(n)))
    return int(n.value)


def dcp_decode_attn_multi_partial(shape: dcp_attn_shape, q_len: int, q, k_cache, v_cache,
                                  block_table, bounds, part_o, part_lse, workspace) -> None:
    _check_attn(shape, q_len, q, k_cache, v_cache, block_table, bounds)
    _check_out(shape, q_len, q.device, part_o=part_o, part_lse=part_lse)
    _check_workspace(workspace, q.device)
    _check(load().dcp_decode_attn_multi_partial(
        ctypes.byref(shape), q_len, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(bounds), _ptr(part_o), _ptr(part_lse), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))


def dcp_decode_attn_multi(shape: dcp_attn_shape, q_len: int, q, k_cache, v_cache, block_table,
                          bounds, workspace, out, out_lse=None) -> None:
    _check_attn(shape, q_len, q, k_cache, v_cache, block_table, bounds)
    _check_out(shape, q_len, q.device, out=out, out_lse=out_lse)
    _check_workspace(workspace, q.device)
    _check(load().dcp_decode_attn_multi(
        ctypes.byref(shape), q_len, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
        _ptr(bounds), _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
        _ptr(out_lse), _stream(q)))


def dcp_read_device_flags(workspace) -> int:
    v = ctypes.c_int32(0)
    _check(load().dcp_read_device_flags(_ptr(workspace), ctypes.byref(v), _stream(workspace)))
    return int(v.value)


def dcp_debug_gather_shard(shape: dcp_attn_shape, cache, block_table, bounds, b: int, s: int,
                           kv_head: int, dst) -> None:
    import torch
    el = _elem(shape)
    heads = 1 if shape.kv_kind == DCP_KV_MLA else shape.num_kv_heads
    _tensor("cache", cache, el,
            min_numel=shape.num_blocks * heads * shape.block_size * shape.head_dim_qk)
    dev = cache.device
    _tensor("block_table", block_table, torch.int32, dev,
            numel=shape.batch * shape.max_blocks_per_seq)
    _tensor("bounds", bounds, torch.int32, dev, numel=shape.batch * shape.num_shards * 2)
    _tensor("dst", dst, el, dev)
    row_elems = shape.head_dim_qk
    max_rows = dst.numel() // row_elems
    _check(load().dcp_debug_gather_shard(
        ctypes.byref(shape), _ptr(cache), _ptr(block_table), _ptr(bounds), b, s, kv_head,
        _ptr(dst), max_rows, _stream(cache)))


def dcp_append_kv(shape: dcp_attn_shape, seq_lens, new_k, new_v, block_table, k_cache, v_cache,
                  owner=None) -> None:
    """Store each request's new row at position seq_lens[b]; owner (int32 [B]) gets the
    owning shard, -1 / -2 for a position without a page / a page outside the pool."""
    import torch
    el = _elem(shape)
    B = shape.batch
    mla = shape.kv_kind == DCP_KV_MLA
    heads = 1 if mla else shape.num_kv_heads
    _tensor("k_cache", k_cache, el,
            min_numel=shape.num_blocks * heads * shape.block_size * shape.head_dim_qk)
    dev = k_cache.device
    _tensor("seq_lens", seq_lens, torch.int32, dev, numel=B)
    _tensor("new_k", new_k, el, dev, numel=B * heads * shape.head_dim_qk)
    if not mla:
        _tensor("new_v", new_v, el, dev, numel=B * heads * shape.head_dim_v)
        _tensor("v_cache", v_cache, el, dev,
                min_numel=shape.num_blocks * heads * shape.block_size * shape.head_dim_v)
    _tensor("block_table", block_table, torch.int32, dev, numel=B * shape.max_blocks_per_seq)
    if owner is not None:
        _tensor("owner", owner, torch.int32, dev, numel=B)
    _check(load().dcp_append_kv(
        ctypes.byref(shape), _ptr(seq_lens), _ptr(new_k), _ptr(new_v), _ptr(block_table),
        _ptr(k_cache), _ptr(v_cache), _ptr(owner), _stream(k_cache)))


def dcp_hbm_read_ceiling(src, sink) -> None:
    """Queue one streaming read of the whole of `src` (a device tensor); `sink` is a device
    int32 tensor with at least 2 x CU-count entries."""
    import torch
    _tensor("src", src, None)
    cus = torch.cuda.get_device_properties(src.device).multi_processor_count
    _tensor("sink", sink, torch.int32, src.device, min_numel=2 * cus)
    _check(load().dcp_hbm_read_ceiling(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                       _stream(src)))


def dcp_kernel_timing_begin(max_launches: int) -> None:
    _check(load().dcp_kernel_timing_begin(max_launches))


def dcp_kernel_timing_end():
    """(launches timed, summed milliseconds) of the partial-attention kernel."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_float(0.0)
    _check(load().dcp_kernel_timing_end(ctypes.byref(n), ctypes.byref(ms)))
    return int(n.value), float(ms.value)
