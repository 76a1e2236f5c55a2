"""Seeded synthetic inputs for sequence-sharded paged decode attention.

This package only draws inputs (context lengths, page pools and block tables,
queries of one or several tokens, KV caches, planted keys, the rows of newly
decoded tokens). It holds none of the attention arithmetic, no shard plan and
no kernel logic; the CPU oracle and the GPU path both consume what it
produces.
"""

from .configs import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_from_f32,
    draw_block_table,
    draw_lengths,
    make_device_inputs,
    make_host_inputs,
    make_new_rows,
    make_queries,
    workload,
)
