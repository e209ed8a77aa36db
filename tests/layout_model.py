"""NumPy model of the library's repacked layout (layout version 1), written from
the layout specification in the library's internal header, independently of the
HIP repack kernel.  Used to check the GPU repack byte for byte.

Spec: block (t, kb) = 16 columns x 128 rows, 1 KiB, block index t*(K/128)+kb;
lane l, word j holds column 16t + l%16, rows 128kb + 32j + 8(l//16) + e (e=0..7),
row e at nibble e//2 + 4*(e%2).  Scales [N/16][K/128][16], row kb holding the
scales of group kb // (group/128); zero-point words [N/16][K/128][2] equal to the
canonical words z[G][2t], z[G][2t+1] of that group.
"""
import numpy as np


def nib_pos(e):
    return e // 2 + 4 * (e % 2)


def repack_codes(Qp: np.ndarray, K: int, N: int) -> np.ndarray:
    U = np.ascontiguousarray(Qp).view(np.uint32)
    T, Gk = N // 16, K // 128
    t = np.arange(T)[:, None, None, None]
    kb = np.arange(Gk)[None, :, None, None]
    l = np.arange(64)[None, None, :, None]
    j = np.arange(4)[None, None, None, :]
    words = U[16 * kb + 4 * j + l // 16, 16 * t + l % 16]
    out = np.zeros_like(words)
    for e in range(8):
        out |= ((words >> np.uint32(4 * e)) & np.uint32(15)) << np.uint32(4 * nib_pos(e))
    return out.reshape(-1)  # uint32, block-major


def repack_scales(s: np.ndarray, N: int, blocks_per_group: int = 1) -> np.ndarray:
    s = np.repeat(s, blocks_per_group, axis=0)
    G = s.shape[0]
    return np.ascontiguousarray(s.reshape(G, N // 16, 16).transpose(1, 0, 2)).reshape(-1)


def repack_zeros(Zp: np.ndarray, N: int, blocks_per_group: int = 1) -> np.ndarray:
    U = np.repeat(np.ascontiguousarray(Zp).view(np.uint32), blocks_per_group, axis=0)
    G = U.shape[0]
    return np.ascontiguousarray(U.reshape(G, N // 16, 2).transpose(1, 0, 2)).reshape(-1)
