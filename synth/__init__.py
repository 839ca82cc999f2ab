"""Seeded synthetic inputs for paged KV-cache attention (shared by the oracle side and the GPU side).

This package draws random numbers and writes down workload structure only: sequence lengths,
the physical-block free order, token K/V values, queries and the allocator-operation script a
workload implies.  It holds none of the method's arithmetic (no slot computation, no gather, no
attention, no fp8 encoding).
"""
from .workloads import (  # noqa: F401
    CONFIG_NAMES, Workload, make_workload, poison_code, elem_bytes, layer_rows, layer_workload,
)
