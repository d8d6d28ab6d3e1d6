"""Seeded synthetic inputs for the KDA decode / verify / commit workloads.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and prepares inputs (normalising q and
k, mapping raw draws to gates in (0, 1), rounding to bf16). It holds none of
the recurrence's arithmetic.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make,
    make_workload,
)
