"""Seeded synthetic inputs for deferred-RoPE paged attention.

This package only draws random numbers and lays them out as the library's
input formats: a block pool of content-only K/V, per-request lists of
(physical block, logical start) entries, queries and new tokens.  It holds
none of the attention arithmetic, imports neither the oracle nor the HIP
binding, and is shared by both sides of every parity test.
"""
from .synth import (  # noqa: F401
    CONFIGS,
    CFG5_PES,
    CFG5_SKEWS,
    WorkloadSpec,
    Workload,
    RequestLayout,
    SparsePool,
    build_workload,
    cache_trace,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    spec,
)
