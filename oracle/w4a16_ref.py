"""Plain CPU definition of the W4A16 GEMM -- TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this module.  It is deliberately slow and obvious: NumPy in float64, no blocking,
no fusion, no reordering beyond what a library matmul does internally.

Pages cited (all three describe the Marlin FP16 x INT4 kernel):
  [P1] "Marlin", Spark Notes, dingiv.github.io/ai/compute/kernel/marlin
  [P2] "Marlin / GPTQ-Marlin", brain.gartu.xyz/ia/llm/quantification/optimisations/marlin/
  [P3] "Marlin Project Overview", vecbase.com/en/p/IST-DASLab/marlin

What is computed ([P2] section "Le problème"): Y = X_fp16 x W_int4, where each
4-bit weight code is turned back into a real weight with the scale (and
zero-point) of its group of 128 consecutive weights along K ([P1] sections
"反量化与 GEMM 融合" and "Group size 为什么是 128"; [P2] section "2. Tiled layout
et repacking").  The value of a weight is w = (q - z) * s, with z = 8 in the
symmetric case.  Converting a 4-bit code to fp16 loses nothing ([P1] section
"反量化精度权衡", point 1); products accumulate in fp32 and the output is fp16
([P1] same section, points 2-3) -- the oracle keeps everything in fp64 instead,
so its result is the exact product up to fp64 rounding of the sum.

Readings where the pages are silent (each is also listed in the design notes):
  * q is packed 8 codes per int32 along K, least-significant nibble first
    (word Qp[i, n], nibble j = row 8i + j); zero-points are packed along N
    (word Zp[G, c], nibble j = column 8c + j).  Words are read as unsigned.
  * Groups are contiguous along K (no act-order permutation); scale s[G, n]
    applies to rows G*g .. G*g + g - 1 of column n.
  * A 2:4-sparse weight is an ordinary weight whose pruned positions carry the
    zero code (q = z), so its oracle is the dense oracle on the pruned codes.
  * W4A8 (fp8 activations, [P1] section "CUTLASS W4A8（混合精度）"): the
    activations are OCP E4M3 codes with an optional fp32 scale per row; the
    product is the same definition on their exact values (decode_e4m3 and
    gemm_w4a8 below).
  * Dequantization inside the matrix unit ([P1] section "与 Blackwell NVFP4 的对比":
    FP4 weights with micro-block scales, turned into real values inside the matrix
    instruction): the FP4 format here is the OCP Microscaling one, MXFP4 -- E2M1
    codes, one E8M0 (power-of-two) scale per 32 consecutive weights along K.  It is
    the micro-block format that gfx950's block-scaled matrix instructions take; the
    page's NVFP4 (E4M3 scales per 16) has no such instruction there.  Codes are
    packed 8 per int32 along K as above; scales E[K/32, N] are bytes.  The
    activations are those of W4A8 (decode_e2m1, decode_e8m0, gemm_mxfp4 below).

Pinned by tests/test_oracle.py (exhaustive nibble tables, exact-rational brute
force, closed forms and invariants); no function here is "parity unpinned".
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional, Sequence, Tuple

import numpy as np


# -- step 1: 4-bit codes of the weights ---------------------------------------
def unpack_codes_k(Qp: np.ndarray, K: int, cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """Codes q[k, n] from words packed along K: q = (Qp[k // 8, n] >> 4*(k % 8)) & 15.

    Returns uint8 [K, N] (or [K, len(cols)] for a column subset).
    """
    U = np.ascontiguousarray(Qp).view(np.uint32)
    if cols is not None:
        U = U[:, np.asarray(cols)]
    assert U.shape[0] * 8 == K
    q = np.empty((K, U.shape[1]), dtype=np.uint8)
    for k in range(8):
        q[k::8] = ((U >> np.uint32(4 * k)) & np.uint32(15)).astype(np.uint8)
    return q


# -- step 2: zero-points ------------------------------------------------------
def unpack_codes_n(Zp: np.ndarray, N: int) -> np.ndarray:
    """Codes z[G, n] from words packed along N: z = (Zp[G, n // 8] >> 4*(n % 8)) & 15."""
    U = np.ascontiguousarray(Zp).view(np.uint32)
    assert U.shape[1] * 8 == N
    z = np.empty((U.shape[0], N), dtype=np.uint8)
    for j in range(8):
        z[:, j::8] = ((U >> np.uint32(4 * j)) & np.uint32(15)).astype(np.uint8)
    return z


def zero_points(G: int, N: int, Zp: Optional[np.ndarray]) -> np.ndarray:
    """z[G, N]: 8 everywhere for the symmetric format, else the unpacked codes."""
    if Zp is None:
        return np.full((G, N), 8, dtype=np.uint8)
    return unpack_codes_n(Zp, N)


# -- step 3: dequantization ---------------------------------------------------
def dequant(Qp: np.ndarray, s: np.ndarray, Zp: Optional[np.ndarray], K: int, N: int,
            group: int, cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """W[k, n] = (q[k, n] - z[k // g, n]) * s[k // g, n] in float64 (exact).

    The product of an integer in [-15, 15] and an fp16 value fits in the 53-bit
    fp64 significand, so this W is the exact real weight.
    """
    assert K % group == 0
    G = K // group
    q = unpack_codes_k(Qp, K, cols).astype(np.float64)
    z = zero_points(G, N, Zp).astype(np.float64)
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
    if cols is not None:
        z = z[:, np.asarray(cols)]
        s64 = s64[:, np.asarray(cols)]
    rows_group = np.arange(K) // group
    return (q - z[rows_group, :]) * s64[rows_group, :]


def dequant_fp16(Qp, s, Zp, K, N, group) -> np.ndarray:
    """fp16 weights W16 = round-to-nearest-even(W): the dequantized matrix the
    unfused baseline writes back to memory before a plain GEMM ([P1] section
    "反量化与 GEMM 融合"; [P2] section "Le problème")."""
    return dequant(Qp, s, Zp, K, N, group).astype(np.float16)


# -- steps 4-5: product and the per-element error scale -----------------------
def gemm(X: np.ndarray, Qp: np.ndarray, s: np.ndarray, Zp: Optional[np.ndarray],
         group: int, rows_per_chunk: int = 1024) -> np.ndarray:
    """Y = X @ W in float64, X given as fp16 [M, K].  Returns float64 [M, N]."""
    M, K = X.shape
    N = Qp.shape[1]
    W = dequant(Qp, s, Zp, K, N, group)
    Y = np.empty((M, N), dtype=np.float64)
    for m0 in range(0, M, rows_per_chunk):
        Y[m0:m0 + rows_per_chunk] = X[m0:m0 + rows_per_chunk].astype(np.float64) @ W
    return Y


def error_bound(X: np.ndarray, Qp: np.ndarray, s: np.ndarray, Zp: Optional[np.ndarray],
                group: int, rows_per_chunk: int = 1024) -> np.ndarray:
    """Bnd[m, n] = sum_k |X[m, k] * W[k, n]|, the scale of the per-element tolerance."""
    M, K = X.shape
    N = Qp.shape[1]
    A = np.abs(dequant(Qp, s, Zp, K, N, group))
    B = np.empty((M, N), dtype=np.float64)
    for m0 in range(0, M, rows_per_chunk):
        B[m0:m0 + rows_per_chunk] = np.abs(X[m0:m0 + rows_per_chunk].astype(np.float64)) @ A
    return B


def gemm_sampled(X: np.ndarray, Qp: np.ndarray, s: np.ndarray, Zp: Optional[np.ndarray],
                 group: int, rows: Sequence[int], cols: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Y and Bnd at the cross product rows x cols only (for full-size shapes)."""
    K = X.shape[1]
    N = Qp.shape[1]
    W = dequant(Qp, s, Zp, K, N, group, cols=cols)
    Xr = X[np.asarray(rows)].astype(np.float64)
    return Xr @ W, np.abs(Xr) @ np.abs(W)


def gemm_exact(X: np.ndarray, Qp: np.ndarray, s: np.ndarray, Zp: Optional[np.ndarray],
               group: int) -> list:
    """Brute-force triple loop in exact rationals (for tiny shapes only).

    Every fp16 input converts exactly to a Fraction, so the result is the real
    value of sum_k X[m,k] * (q[k,n] - z[G,n]) * s[G,n] with no rounding at all.
    Codes are extracted bit by bit from Python integers, independently of the
    NumPy unpack above.
    """
    M, K = X.shape
    N = Qp.shape[1]
    Qw = [[int(v) & 0xFFFFFFFF for v in row] for row in np.asarray(Qp, dtype=np.int64)]
    Zw = None if Zp is None else [[int(v) & 0xFFFFFFFF for v in row] for row in np.asarray(Zp, dtype=np.int64)]
    Xf = [[Fraction(float(v)) for v in row] for row in np.asarray(X, dtype=np.float16)]
    Sf = [[Fraction(float(v)) for v in row] for row in np.asarray(s, dtype=np.float16)]
    Y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                word = Qw[k // 8][n]
                q = 0
                for b in range(4):
                    q |= ((word >> (4 * (k % 8) + b)) & 1) << b
                G = k // group
                if Zw is None:
                    z = 8
                else:
                    zw = Zw[G][n // 8]
                    z = 0
                    for b in range(4):
                        z |= ((zw >> (4 * (n % 8) + b)) & 1) << b
                acc += Xf[m][k] * (q - z) * Sf[G][n]
            Y[m][n] = acc
    return Y


# -- W4A8: fp8 (E4M3) activations ---------------------------------------------
# [P1] section "CUTLASS W4A8（混合精度）" describes the neighbouring variant: INT4
# weights times FP8 activations, so that the matrix product runs on FP8 matrix
# units.  The pages fix neither the FP8 encoding nor how activations are scaled.
# Readings taken: activations arrive as OCP FP8 E4M3 codes (the encoding of
# the "FP8" of that section's hardware; 1 sign bit, 4 exponent bits with bias
# 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448),
# with an optional fp32 scale per activation row (None means 1); the weights
# are the same (q - z) * s as above and the output is fp16.
def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """Real values (float64) of OCP E4M3 byte codes.

    exponent field e = 0: (-1)^sign * 2^-6 * m/8 (subnormal);
    otherwise:            (-1)^sign * 2^(e-7) * (1 + m/8);
    e = 15 and m = 7:     NaN.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    v = sign * np.where(e == 0, sub, normal)
    return np.where((e == 15) & (c & 7 == 7), np.nan, v)


def activations_w4a8(X8: np.ndarray, xscale: Optional[np.ndarray]) -> np.ndarray:
    """Activation values a[m] * x[m, k] in float64 (exact: a 24-bit times a
    4-bit significand fits in 53 bits)."""
    Xv = decode_e4m3(X8)
    if xscale is not None:
        Xv = Xv * np.asarray(xscale, dtype=np.float32).astype(np.float64)[:, None]
    return Xv


def gemm_w4a8(X8: np.ndarray, xscale: Optional[np.ndarray], Qp: np.ndarray, s: np.ndarray,
              Zp: Optional[np.ndarray], group: int) -> np.ndarray:
    """Y[m, n] = a[m] * sum_k x8[m, k] * (q[k, n] - z) * s[k // g, n], float64 [M, N]."""
    K = X8.shape[1]
    N = Qp.shape[1]
    return activations_w4a8(X8, xscale) @ dequant(Qp, s, Zp, K, N, group)


def error_bound_w4a8(X8: np.ndarray, xscale: Optional[np.ndarray], Qp: np.ndarray,
                     s: np.ndarray, Zp: Optional[np.ndarray], group: int) -> np.ndarray:
    """Bnd[m, n] = sum_k |a[m] * x8[m, k] * W[k, n]|."""
    K = X8.shape[1]
    N = Qp.shape[1]
    return np.abs(activations_w4a8(X8, xscale)) @ np.abs(dequant(Qp, s, Zp, K, N, group))


def gemm_w4a8_sampled(X8, xscale, Qp, s, Zp, group, rows, cols):
    """Y and Bnd of the W4A8 product at the cross product rows x cols only."""
    K = X8.shape[1]
    N = Qp.shape[1]
    W = dequant(Qp, s, Zp, K, N, group, cols=cols)
    r = np.asarray(rows)
    Xr = activations_w4a8(X8[r], None if xscale is None else np.asarray(xscale)[r])
    return Xr @ W, np.abs(Xr) @ np.abs(W)


# -- MXFP4 weights (dequantization inside the matrix instruction) ---------------
def decode_e2m1(codes: np.ndarray) -> np.ndarray:
    """Real values (float64) of OCP E2M1 4-bit codes (OCP Microscaling Formats v1.0,
    FP4 element): sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0.

    exponent field e = 0: (-1)^sign * m/2 (subnormal: 0 or 0.5);
    otherwise:            (-1)^sign * 2^(e-1) * (1 + m/2).
    No infinities or NaN: the 16 codes are +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    """
    c = np.asarray(codes).astype(np.int64) & 15
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64))
    return sign * np.where(e == 0, m / 2.0, normal)


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """Real values (float64) of OCP E8M0 scale bytes: 2^(e - 127), e = 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def dequant_mxfp4(Qp: np.ndarray, E: np.ndarray, K: int, N: int,
                  cols: Optional[Sequence[int]] = None) -> np.ndarray:
    """W[k, n] = e2m1(q[k, n]) * 2^(E[k // 32, n] - 127) in float64 (exact)."""
    q = unpack_codes_k(Qp, K, cols)
    Ec = E if cols is None else E[:, np.asarray(cols)]
    scale = np.repeat(decode_e8m0(Ec), 32, axis=0)
    return decode_e2m1(q) * scale


def gemm_mxfp4(X8: np.ndarray, xscale: Optional[np.ndarray], Qp: np.ndarray,
               E: np.ndarray) -> np.ndarray:
    """Y[m, n] = a[m] * sum_k x8[m, k] * e2m1(q[k, n]) * 2^(E[k // 32, n] - 127),
    float64 [M, N]; x8 are E4M3 activation codes with optional fp32 row scales a."""
    K = X8.shape[1]
    N = Qp.shape[1]
    return activations_w4a8(X8, xscale) @ dequant_mxfp4(Qp, E, K, N)


def error_bound_mxfp4(X8: np.ndarray, xscale: Optional[np.ndarray], Qp: np.ndarray,
                      E: np.ndarray) -> np.ndarray:
    """Bnd[m, n] = sum_k |a[m] * x8[m, k] * W[k, n]|."""
    K = X8.shape[1]
    N = Qp.shape[1]
    return np.abs(activations_w4a8(X8, xscale)) @ np.abs(dequant_mxfp4(Qp, E, K, N))


def gemm_mxfp4_sampled(X8, xscale, Qp, E, rows, cols):
    """Y and Bnd of the MXFP4 product at the cross product rows x cols only."""
    K = X8.shape[1]
    N = Qp.shape[1]
    W = dequant_mxfp4(Qp, E, K, N, cols=cols)
    r = np.asarray(rows)
    Xr = activations_w4a8(X8[r], None if xscale is None else np.asarray(xscale)[r])
    return Xr @ W, np.abs(Xr) @ np.abs(W)


# -- step 6: acceptance -------------------------------------------------------
def accept(Y: np.ndarray, Yref: np.ndarray, Bnd: np.ndarray, rel_fro: float = 1e-3,
           elem_rel: float = 5e-3, elem_abs: float = 1e-4) -> Tuple[bool, dict]:
    """Accept a computed fp16 result Y against the fp64 oracle.

    Y passes when every element is finite, the relative Frobenius error is at
    most rel_fro (skipped when the reference is exactly zero) and every element
    obeys |Y - Yref| <= elem_rel * Bnd + elem_abs.  fp32 accumulation over K,
    one rounding of W to fp16 and one rounding of Y to fp16 each stay well
    inside elem_rel * Bnd for K up to 28672 (see the design notes).
    """
    Y64 = np.asarray(Y).astype(np.float64)
    info = {}
    finite = bool(np.all(np.isfinite(Y64)))
    info["finite"] = finite
    err = np.abs(Y64 - Yref)
    ref_norm = float(np.linalg.norm(Yref))
    fro = float(np.linalg.norm(Y64 - Yref)) / ref_norm if ref_norm > 0 else 0.0
    info["rel_fro"] = fro
    lim = elem_rel * Bnd + elem_abs
    ratio = err / lim
    info["max_err_over_limit"] = float(np.nanmax(ratio)) if ratio.size else 0.0
    info["max_abs_err"] = float(np.nanmax(err)) if err.size else 0.0
    ok = finite and (ref_norm == 0 or fro <= rel_fro) and bool(np.all(err <= lim))
    return ok, info


# -- 2:4 structure --------------------------------------------------------------
def check_24(Qp: np.ndarray, K: int, Zp: Optional[np.ndarray] = None, group: int = 128) -> bool:
    """True when every aligned run of 4 consecutive K in every column holds at
    least 2 zero weights (code equal to the zero-point), the structure that 2:4
    sparse tensor cores require ([P1] section "支持 2:4 稀疏加速"; [P2] section
    "4. Support de la sparsité 2:4")."""
    N = Qp.shape[1]
    q = unpack_codes_k(Qp, K)
    z = zero_points(K // group, N, Zp)[np.arange(K) // group, :]
    zero = (q == z).reshape(K // 4, 4, N).sum(axis=1)
    return bool(np.all(zero >= 2))
