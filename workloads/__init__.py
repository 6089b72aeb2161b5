"""Seeded synthetic inputs for row-wise top-k selection.

This package only draws numbers: it holds none of the selection arithmetic.
Both the CPU oracle side (tests, CPU baseline) and the GPU side (tests, bench)
take their inputs from here, so the two sides read the same bytes.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    make_workload,
    make_edge_rows,
    pad_rows,
)
