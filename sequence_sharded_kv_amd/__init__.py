"""Sequence-sharded paged decode attention (the DCP decode hot path) for MI355X.

The compute lives in libdcp.so (HIP kernels for gfx950 behind the C ABI in
include/dcp.h); this package is its ctypes binding. Build the library with
``python -m sequence_sharded_kv_amd._build``.
"""

from ._lib import (  # noqa: F401
    DCP_BF16,
    DCP_ERR_ALIGN,
    DCP_ERR_BAD_PLAN,
    DCP_ERR_DEVICE,
    DCP_ERR_NULL,
    DCP_ERR_SHAPE,
    DCP_ERR_UNSUPPORTED,
    DCP_ERR_WORKSPACE,
    DCP_F32,
    DCP_KV_GQA,
    DCP_KV_MLA,
    DCP_NOALLOC_SCRATCH_BYTES,
    DCP_OK,
    EXPORTS,
    LIB_PATH,
    DcpError,
    dcp_abi_version,
    dcp_append_kv,
    dcp_attn_shape,
    dcp_debug_gather_shard,
    dcp_decode_attn,
    dcp_decode_attn_multi,
    dcp_decode_attn_multi_partial,
    dcp_decode_attn_noalloc,
    dcp_decode_attn_partial,
    dcp_hbm_read_ceiling,
    dcp_kernel_timing_begin,
    dcp_kernel_timing_end,
    dcp_last_error,
    dcp_merge_lse,
    dcp_plan_shards,
    dcp_plan_shards_device,
    dcp_read_device_flags,
    dcp_status_string,
    dcp_workspace_bytes,
    dcp_workspace_bytes_multi,
    load,
    make_shape,
)


def alloc_workspace(shape, device, q_len: int = 1):
    """One workspace for `shape` and `q_len` query tokens per request (reuse it across calls;
    see dcp_workspace_bytes / dcp_workspace_bytes_multi)."""
    import torch
    n = dcp_workspace_bytes_multi(shape, q_len)
    return torch.empty(n, dtype=torch.uint8, device=device)
