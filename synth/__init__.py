"""Seeded synthetic inputs for the MLA prolog (shared by the oracle tests, the
GPU tests and the benchmark).

This package draws random numbers and lays them out in the shapes and dtypes of
the MLA prolog operator's inputs; it performs none of the operator's arithmetic.
"""
from .generate import (  # noqa: F401
    Dims, Workload, WORKLOADS, make_inputs, workload, bf16_bits_to_f32,
    SENTINEL_BF16, SENTINEL_F16, SENTINEL_I8,
)
