"""Helpers for the GPU tests: move seeded inputs to the device and run the
library through its Python binding (which calls the C ABI)."""
import numpy as np
import torch

import w4a16_mixed_precision_offline_amd as w4


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def repack(d: dict, K: int, N: int, group: int = 128):
    """Canonical weights dict (from gen.weights) -> device (wp, sp, zp)."""
    q = dev(d["Qp"])
    s = dev(d["s"])
    z = dev(d["Zp"]) if d.get("Zp") is not None else None
    wp, sp, zp = w4.alloc_packed(K, N, group, z is not None)
    w4.w4a16_repack(q, s, z, wp, sp, zp, K, N, group)
    return wp, sp, zp


def gemm(X: torch.Tensor, packed, M, N, K, group=128, variant=-1, splits=0, Y=None):
    wp, sp, zp = packed
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    if variant == -1 and splits == 0:
        w4.w4a16_gemm(X, wp, sp, zp, Y, M, N, K, group)
    else:
        w4.w4a16_gemm_plan(X, wp, sp, zp, Y, M, N, K, group, variant, splits)
    return Y


def nan_filled(M, N):
    return torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")


def variant_index(name: str) -> int:
    for v in range(w4.w4a16_gemm_variants()):
        if w4.w4a16_gemm_variant_name(v) == name:
            return v
    raise KeyError(name)


def tile_samples(M: int, N: int):
    """One row in every 16-row tile and one column in every 16-column tile (at a
    position that moves through the tile from one tile to the next), plus the last row
    and column: comparing Y on this cross product against the oracle reaches every
    output tile of every kernel (16 x 16 matrix tiles and everything built from them),
    every wave's columns and every stream-K piece."""
    rows = sorted({min(M - 1, 16 * i + (7 * i) % 16) for i in range((M + 15) // 16)} | {M - 1})
    cols = sorted({16 * j + (5 * j) % 16 for j in range(N // 16)} | {N - 1})
    return rows, cols
