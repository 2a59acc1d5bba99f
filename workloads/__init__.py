"""Seeded synthetic workloads for the token-block pruning path.

This package only builds inputs (packed lengths, Q/K tensors with planted
blocks, hidden states, positions).  It holds none of the pruning arithmetic,
so both the CPU oracle and the GPU library can be fed from it without
sharing any of the method's code.
"""
from .gen import (  # noqa: F401
    splitmix64_py,
    stream_key,
    draw_u64,
    uniform53,
    normal,
    Workload,
    WORKLOADS,
    get_workload,
    make_lengths,
    make_inputs,
    cu_from_lengths,
)
