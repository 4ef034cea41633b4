"""Seeded synthetic inputs for the MoE expert-parallel layout / dispatch / combine path.

This package only draws inputs (hidden rows, top-k routing, route weights,
shared-expert outputs, stand-in expert outputs).  It holds none of the path's
own arithmetic: no histogram, scan, permutation, quantisation or weighted sum.
Both the GPU path's tests and the CPU oracle's tests consume the same bytes
from here.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    WorkloadConfig,
    make_workload,
    normal_bf16_bits,
    random_expert_out_bits,
    stamped_rows_bf16_bits,
    uniform_distinct_routing,
    group_limited_routing,
    zipf_routing,
    softmax_weights,
    maxvio,
    PAD_NONE,
    PAD_MULTIPLE,
    PAD_CAPACITY,
)
