"""Seeded synthetic workloads for the W4A16 GEMM.

Workload shapes and value distributions follow the five benchmark configurations
of this project (tiny 1024x1024; the 7B-class decode sweep; the 70B-class large
layers; the zero-point / awkward-shape set; the 2:4-sparse set).  The pages that
describe the method (Marlin, on dingiv.github.io, brain.gartu.xyz and
vecbase.com) name Llama-2-class models and GPTQ/AWQ checkpoints; no weights or
datasets are used here, only the layer shapes, with synthetic values.

Storage format produced here (the library's canonical input):
  * q  : 4-bit codes 0..15, shape [K, N]; packed along K into int32 words
         Qp[K/8, N], nibble j (bits 4j..4j+3) of Qp[i, n] holds row 8i+j.
  * s  : fp16 scales, shape [K/g, N] (one per group of g consecutive K, per column).
  * z  : 4-bit zero-points, shape [K/g, N]; packed along N into Zp[K/g, N/8],
         nibble j of Zp[G, c] holds column 8c+j.  Symmetric runs use z = 8 and
         pass no Zp.
  * X  : fp16 activations, shape [M, K], row-major.

Random draws use numpy's PCG64 bit generator with a seed derived from the
configuration and shape, so that every M of one (cfg, K, N) shares its weights.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

GROUP = 128


@dataclass(frozen=True)
class Workload:
    cfg: int
    M: int
    K: int
    N: int
    group: int = GROUP
    asym: bool = False
    sparse24: bool = False
    s_lo: float = 0.002
    s_hi: float = 0.02

    @property
    def name(self) -> str:
        kind = "asym" if self.asym else ("2:4" if self.sparse24 else "sym")
        return f"c{self.cfg}:{kind}:M{self.M}:K{self.K}:N{self.N}:g{self.group}"


# The five benchmark configurations: (K, N) list, M list, and value recipe.
CONFIGS: Dict[int, dict] = {
    0: dict(KN=[(1024, 1024)], Ms=[16], asym=False, sparse24=False, s=(0.002, 0.02),
            title="Tiny W4A16 GEMM"),
    1: dict(KN=[(4096, 4096), (4096, 12288), (4096, 11008), (11008, 4096)],
            Ms=[1, 2, 4, 8, 16, 32], asym=False, sparse24=False, s=(0.002, 0.02),
            title="Decode-shape sweep, 7B-class linear layers"),
    2: dict(KN=[(8192, 28672), (28672, 8192), (8192, 10240)],
            Ms=[16, 64, 256, 1024, 4096], asym=False, sparse24=False, s=(0.001, 0.01),
            title="Large-layer sweep, 70B-class shapes"),
    3: dict(KN=[(2560, 2560), (5120, 13824), (13824, 5120), (3072, 768)],
            Ms=[1, 16, 48, 128], asym=True, sparse24=False, s=(0.002, 0.02),
            title="Asymmetric (zero-point) and awkward shapes"),
    4: dict(KN=[(4096, 4096), (8192, 28672)], Ms=[16, 32, 128], asym=False,
            sparse24=True, s=(0.002, 0.02), title="2:4-structured-sparse INT4"),
}


def config_runs(cfg: int) -> List[Workload]:
    c = CONFIGS[cfg]
    out = []
    for (K, N) in c["KN"]:
        for M in c["Ms"]:
            out.append(Workload(cfg=cfg, M=M, K=K, N=N, asym=c["asym"],
                                sparse24=c["sparse24"], s_lo=c["s"][0], s_hi=c["s"][1]))
    return out


def seed_for_weights(cfg: int, K: int, N: int) -> int:
    return 1_000_003 * cfg + 101 * K + N


def seed_for_activations(cfg: int, M: int, K: int, N: int) -> int:
    return 1_000_003 * cfg + 10_007 * M + 101 * K + N


def pack_nibbles_along_k(q: np.ndarray) -> np.ndarray:
    """[K, N] codes 0..15 -> [K/8, N] int32; nibble j of word i holds row 8i+j."""
    K, N = q.shape
    assert K % 8 == 0
    acc = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        acc |= q[j::8].astype(np.uint32) << np.uint32(4 * j)
    return acc.view(np.int32)


def pack_nibbles_along_n(z: np.ndarray) -> np.ndarray:
    """[G, N] codes 0..15 -> [G, N/8] int32; nibble j of word c holds column 8c+j."""
    G, N = z.shape
    assert N % 8 == 0
    acc = np.zeros((G, N // 8), dtype=np.uint32)
    for j in range(8):
        acc |= z[:, j::8].astype(np.uint32) << np.uint32(4 * j)
    return acc.view(np.int32)


# The six ways to keep 2 of 4 positions, ascending.
KEEP_PAIRS = np.array([(0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3)], dtype=np.int64)


def weights(w: Workload, seed: Optional[int] = None) -> dict:
    """Quantized weights for workload `w`.

    Returns a dict with q (uint8 [K,N]), Qp (int32 [K/8,N]), s (fp16 [G,N]),
    z (uint8 [G,N] or None), Zp (int32 [G,N/8] or None) and, for 2:4 runs,
    keep (bool [K,N]): True where a weight was kept, False where it was forced
    to the zero code (q = 8).
    """
    K, N, g = w.K, w.N, w.group
    assert K % g == 0 and K % 8 == 0 and N % 8 == 0
    G = K // g
    rng = np.random.Generator(np.random.PCG64(seed_for_weights(w.cfg, K, N) if seed is None else seed))
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    s = rng.uniform(w.s_lo, w.s_hi, size=(G, N)).astype(np.float32).astype(np.float16)
    z = None
    Zp = None
    if w.asym:
        z = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
        Zp = pack_nibbles_along_n(z)
    keep = None
    if w.sparse24:
        assert not w.asym, "2:4 runs are symmetric"
        assert K % 4 == 0
        pat = rng.integers(0, 6, size=(K // 4, N))
        keep = np.zeros((K // 4, 4, N), dtype=bool)
        a = KEEP_PAIRS[pat, 0]
        b = KEEP_PAIRS[pat, 1]
        for p in range(4):
            keep[:, p, :] = (a == p) | (b == p)
        keep = keep.reshape(K, N)
        q = np.where(keep, q, np.uint8(8)).astype(np.uint8)
    Qp = pack_nibbles_along_k(q)
    return dict(q=q, Qp=Qp, s=s, z=z, Zp=Zp, keep=keep)


def activations(w: Workload, seed: Optional[int] = None) -> np.ndarray:
    """X [M, K] fp16: N(0,1) drawn in fp32, rounded to nearest-even fp16."""
    rng = np.random.Generator(np.random.PCG64(
        seed_for_activations(w.cfg, w.M, w.K, w.N) if seed is None else seed))
    return rng.standard_normal((w.M, w.K), dtype=np.float32).astype(np.float16)


def activations_bf16(w: Workload, seed: Optional[int] = None):
    """X [M, K] bf16 for the bf16-activation entry points: N(0,1) drawn in fp32, rounded
    to nearest-even bf16.  Returns (bits uint16 [M, K], values float32 [M, K])."""
    rng = np.random.Generator(np.random.PCG64(
        seed_for_activations(w.cfg, w.M, w.K, w.N) if seed is None else seed))
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)



def activations_fp8(w: Workload, seed: Optional[int] = None):
    """X [M, K] as OCP FP8 E4M3 codes with one fp32 scale per row, for the W4A8 entry
    points: x ~ N(0,1) drawn in fp32 (the same draw as `activations`), a[m] = max_k
    |x[m, k]| / 448 (448 is the largest finite E4M3 value), codes = the E4M3 value
    nearest to x / a (ties to even; torch's float8_e4m3fn cast).  This is the caller's
    per-row quantization of its activations, not a step of the method.
    Returns (codes uint8 [M, K], a float32 [M])."""
    import torch

    rng = np.random.Generator(np.random.PCG64(
        seed_for_activations(w.cfg, w.M, w.K, w.N) if seed is None else seed))
    x = rng.standard_normal((w.M, w.K), dtype=np.float32)
    amax = np.abs(x).max(axis=1) if w.K else np.zeros(w.M, np.float32)
    a = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    xs = torch.from_numpy(x / a[:, None])
    codes = xs.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, a


def weights_mxfp4(w: Workload, seed: Optional[int] = None) -> dict:
    """MXFP4 weights for the block-scaled entry points: E2M1 codes uniform over all
    16 (every code is a valid value) packed 8 per int32 along K like the 4-bit
    codes of `weights`, and one E8M0 scale byte per 32 rows of a column, uniform in
    [119, 124] (scales 2^-8 .. 2^-3: weights up to 6 * 2^-3, the range of the
    group-quantized weights).  Returns {"q": uint8 [K, N], "Qp": int32 [K/8, N],
    "E": uint8 [K/32, N]}."""
    rng = np.random.Generator(np.random.PCG64(
        seed_for_weights(w.cfg, w.K, w.N) + 17 if seed is None else seed))
    q = rng.integers(0, 16, size=(w.K, w.N), dtype=np.uint8)
    E = rng.integers(119, 125, size=(w.K // 32, w.N), dtype=np.uint8)
    return {"q": q, "Qp": pack_nibbles_along_k(q), "E": E}
