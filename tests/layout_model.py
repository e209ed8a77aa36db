"""NumPy model of the library's repacked layout (layout version 1), written from
the layout specification in the library's internal header, independently of the
HIP repack kernel.  Used to check the GPU repack byte for byte.

Spec: block (t, kb) = 16 columns x 128 rows, 1 KiB, block index t*(K/128)+kb;
lane l, word j holds column 16t + l%16, rows 128kb + 32j + 8(l//16) + e (e=0..7),
row e at nibble e//2 + 4*(e%2).  Scales [N/16][K/128][16], row kb holding the
scales of group kb // (group/128); zero-point words [N/16][K/128][2] equal to the
canonical words z[G][2t], z[G][2t+1] of that group.  Groups of 64 rows: two scale
rows per block interleaved per column ([N/16][K/128][16][2]) and two zero-point
word pairs per block ([N/16][K/128][2][2]), half h = rows 64h .. 64h+63.
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


def repack_scales64(s: np.ndarray, N: int) -> np.ndarray:
    """Groups of 64 rows: [N/16][K/128][16 columns][2 halves], half h of block kb holding
    group 2kb + h."""
    G = s.shape[0]
    return np.ascontiguousarray(s.reshape(G // 2, 2, N // 16, 16).transpose(2, 0, 3, 1)).reshape(-1)


def repack_zeros64(Zp: np.ndarray, N: int) -> np.ndarray:
    """Groups of 64 rows: [N/16][K/128][2 halves][2 words], half h of block kb holding the
    canonical words z[2kb + h][2t], z[2kb + h][2t + 1]."""
    U = np.ascontiguousarray(Zp).view(np.uint32)
    G = U.shape[0]
    return np.ascontiguousarray(U.reshape(G // 2, 2, N // 16, 2).transpose(2, 0, 1, 3)).reshape(-1)


# ---- 2:4 sparse layout -------------------------------------------------------------
# Per (tile t, block kb), lane l owns column 16t + l%16 and, for half h, the dense rows
# 128kb + 64h + 16(l//16) + [0, 16) = four aligned runs g of 4.  From each run it keeps
# two positions (the non-zero codes, topped up with the lowest free positions,
# ascending) as elements 2g, 2g+1 of a word (element e at nibble e//2 + 4(e%2)); the
# positions are 2-bit fields at bits 16h + 2e of the lane's metadata word.
def _keep_table():
    table = {}
    for mask in range(16):
        nz = [p for p in range(4) if mask >> p & 1]
        if len(nz) > 2:
            table[mask] = None
            continue
        keep = list(nz)
        for p in range(4):
            if len(keep) == 2:
                break
            if p not in keep:
                keep.append(p)
        table[mask] = tuple(sorted(keep))
    return table


def sparse24_compress(q: np.ndarray, K: int, N: int):
    """q: codes [K, N] (uint8), every aligned run of 4 along K with <= 2 codes != 8.
    Returns (vp uint32 [N/16, K/128, 64, 2], meta uint32 [N/16, K/128, 64])."""
    T, Gk = N // 16, K // 128
    table = _keep_table()
    vp = np.zeros((T, Gk, 64, 2), dtype=np.uint32)
    meta = np.zeros((T, Gk, 64), dtype=np.uint32)
    for h in range(2):
        for qg in range(4):          # lane group l // 16
            for g in range(4):
                rows = (np.arange(Gk)[:, None] * 128 + 64 * h + 16 * qg + 4 * g +
                        np.arange(4)[None, :])                      # [Gk, 4]
                codes = q[rows.reshape(-1), :].reshape(Gk, 4, T, 16)  # [Gk, p, T, c]
                mask = sum(((codes[:, p] != 8).astype(np.int64) << p) for p in range(4))  # [Gk, T, c]
                assert all(table[m] is not None for m in np.unique(mask)), "not 2:4"
                keep = np.array([table[m] for m in range(16)], dtype=object)
                k0 = np.vectorize(lambda m: table[m][0])(mask)
                k1 = np.vectorize(lambda m: table[m][1])(mask)
                for u, kk in ((0, k0), (1, k1)):
                    e = 2 * g + u
                    c = np.take_along_axis(codes, kk[:, None], axis=1)[:, 0]   # [Gk, T, c]
                    lanes = 16 * qg + np.arange(16)
                    vp[:, :, lanes, h] |= (c.transpose(1, 0, 2).astype(np.uint32)
                                           << np.uint32(4 * nib_pos(e)))
                    meta[:, :, lanes] |= (kk.transpose(1, 0, 2).astype(np.uint32)
                                          << np.uint32(16 * h + 2 * e))
    return vp, meta


def mx_repack(Qp: np.ndarray, E: np.ndarray, K: int, N: int):
    """The MXFP4 layout, written as loops over the documented index map: code block
    (t, kb) of 1 KiB, lane l, word w = canonical word kb*16 + 4(l//16) + w of column
    16t + l%16; scale block (t, kb) of 64 bytes, byte l = E[kb*4 + l//16, 16t + l%16]."""
    T, Gk = N // 16, K // 128
    words = np.zeros((T, Gk, 64, 4), dtype=np.uint32)
    scales = np.zeros((T, Gk, 64), dtype=np.uint8)
    Qu = Qp.view(np.uint32)
    for t in range(T):
        for kb in range(Gk):
            for l in range(64):
                col = 16 * t + l % 16
                for w in range(4):
                    words[t, kb, l, w] = Qu[kb * 16 + 4 * (l // 16) + w, col]
                scales[t, kb, l] = E[kb * 4 + l // 16, col]
    return words.reshape(-1), scales.reshape(-1)
