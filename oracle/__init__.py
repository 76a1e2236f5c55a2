"""Float64 CPU oracle (test infrastructure only; see oracle.oracle)."""

from .oracle import (  # noqa: F401
    as_f64,
    attention,
    bf16_bits_to_f64,
    full_attention,
    gather_gqa,
    gather_mla,
    merge_lse,
    partial_attention,
    plan_shards,
    sharded_attention,
)
