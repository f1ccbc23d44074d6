"""Seeded synthetic inputs for the compressed-KV decode workloads.

This package is shared by the CPU oracle side (tests, the CPU baseline) and the GPU
harness (tests, bench).  It holds no attention, RoPE, pooling or selection
arithmetic: only a counter-based generator of approximately N(0,1) values, the
rounding of those values to the storage dtype, and the workload shapes.

Every value is a pure function of (seed, tag, element index), so any slice of any
tensor of any workload can be regenerated on the CPU without materialising the
whole tensor, and the GPU-side generator produces bit-identical values.
"""
from .gen import (  # noqa: F401
    NormalStream,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    hash_positions,
    mix32,
    quantile_table,
    stream_key,
)
from .workloads import WORKLOADS, Workload  # noqa: F401
