"""Seeded synthetic inputs shaped like the VAR-Q workloads.

This package is shared by the tests, the benchmark and the smoke check. It holds
no quantizer, packing or attention arithmetic: it only draws random tensors with
the channel x block outlier structure the VAR-Q project page describes, and it
describes the block schedules (group boundaries) of each workload.
"""

from .kv_synth import (  # noqa: F401
    INFINITY_1024_SIDES,
    VAR_SIDES,
    Workload,
    WORKLOADS,
    frame_offsets,
    gen_next_scale_kv,
    gen_pre_rope_frame_k,
    gen_queries,
    gen_rope_frame_k,
    gen_unit_v,
    rope_frame_tables,
    scale_offsets,
    workload_inputs,
)
