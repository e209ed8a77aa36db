"""CPU oracle for the W4A16 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the test suite (tests/), the smoke check in __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call anything in this package.  The
library and its Python binding never do: the product path runs entirely in the
HIP kernels and fails loudly when they are missing.

The oracle shares no code with the HIP path.  See w4a16_ref.py for the
definitions it implements and the passages they follow.
"""
from .w4a16_ref import (  # noqa: F401
    accept,
    activations_w4a8,
    decode_e2m1,
    decode_e4m3,
    decode_e8m0,
    dequant_mxfp4,
    check_24,
    dequant,
    dequant_fp16,
    error_bound,
    error_bound_mxfp4,
    error_bound_w4a8,
    gemm,
    gemm_exact,
    gemm_mxfp4,
    gemm_mxfp4_sampled,
    gemm_sampled,
    gemm_w4a8,
    gemm_w4a8_sampled,
    unpack_codes_k,
    unpack_codes_n,
    zero_points,
)
