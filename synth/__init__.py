"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This package holds no arithmetic of the sparse-attention method itself: it only draws
Q/K/V tensors (and decode caches) with the shapes and structure of the workloads the
pages measure on, and rounds them once to bfloat16.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    PrefillInputs,
    DecodeInputs,
    make_prefill,
    make_decode,
    bf16_round_bits,
    bf16_bits_to_f32,
    bf16_bits_to_f64,
)
