"""Seeded synthetic inputs for the W4A16 GEMM (shared by tests, smoke and bench).

This package produces inputs only: activations, 4-bit weight codes, fp16 scales,
4-bit zero-points, 2:4 keep-masks, MXFP4 codes and E8M0 scale bytes, plus the canonical packing of the 4-bit
codes into int32 words (the storage format the library accepts).  It holds none
of the method's arithmetic: no dequantization, no matrix product, no repack.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    Workload,
    activations,
    activations_bf16,
    activations_fp8,
    config_runs,
    pack_nibbles_along_k,
    pack_nibbles_along_n,
    seed_for_activations,
    seed_for_weights,
    weights,
    weights_mxfp4,
)
