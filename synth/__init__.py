"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package draws random numbers and stores them in the byte formats the
indexer consumes.  It performs no step of the indexer's own arithmetic
(no dot products, no ReLU, no head reduction, no selection), so the oracle
and the HIP path stay independent of each other even though they read the
same bytes.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    make_rng,
    to_bf16_bits,
    quantize_fp8_rows,
    softmax_weights,
    prefill_inputs,
    decode_inputs,
    tie_heavy_prefill,
    config_inputs,
)
