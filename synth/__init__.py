"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.  This package draws random numbers and rounds them to storage
dtypes; it holds none of the transposed-convolution arithmetic."""

from .inputs import (  # noqa: F401
    SEED,
    round_to_dtype,
    bf16_bits,
    f16_bits,
    uniform,
    normal,
    istft_basis,
    WORKLOADS,
    workload,
)
