"""CPU self-checks of the NumPy layout model used to verify the GPU repack."""
import numpy as np

import layout_model as lm


def test_model_is_a_bijection_on_words():
    # words whose 8 nibbles are equal are unchanged by the nibble permutation, so the
    # multiset of words must be preserved exactly
    K, N = 256, 32
    base = (np.arange(K // 8 * N, dtype=np.uint32) % 16).reshape(K // 8, N)
    Qp = (base * np.uint32(0x11111111)).view(np.int32)
    out = lm.repack_codes(Qp, K, N)
    assert sorted(out.tolist()) == sorted(Qp.view(np.uint32).reshape(-1).tolist())


def test_model_places_rows_as_specified():
    # code of (k, n) = (k + 3n) % 16; read it back from the model through the spec
    K, N = 256, 32
    q = np.array([[(k + 3 * n) % 16 for n in range(N)] for k in range(K)], dtype=np.uint8)
    from gen import pack_nibbles_along_k
    out = lm.repack_codes(pack_nibbles_along_k(q), K, N).reshape(N // 16, K // 128, 64, 4)
    for t in range(N // 16):
        for kb in range(K // 128):
            for l in range(64):
                for j in range(4):
                    w = int(out[t, kb, l, j])
                    for e in range(8):
                        k = 128 * kb + 32 * j + 8 * (l // 16) + e
                        n = 16 * t + l % 16
                        assert (w >> (4 * lm.nib_pos(e))) & 15 == q[k, n]


def test_scale_and_zero_models():
    G, N = 3, 48
    s = np.arange(G * N, dtype=np.uint16).reshape(G, N).view(np.float16)
    sp = lm.repack_scales(s, N).view(np.uint16).reshape(N // 16, G, 16)
    for t in range(N // 16):
        for g in range(G):
            assert list(sp[t, g]) == [g * N + 16 * t + c for c in range(16)]
    Zp = np.arange(G * N // 8, dtype=np.uint32).reshape(G, N // 8).view(np.int32)
    zp = lm.repack_zeros(Zp, N).reshape(N // 16, G, 2)
    for t in range(N // 16):
        for g in range(G):
            assert list(zp[t, g]) == [g * (N // 8) + 2 * t, g * (N // 8) + 2 * t + 1]


def test_scale_and_zero_models_group64():
    # two rows per 128-row block: half h of block kb holds group 2kb + h
    Gk, N = 3, 48
    G = 2 * Gk
    s = np.arange(G * N, dtype=np.uint16).reshape(G, N).view(np.float16)
    sp = lm.repack_scales64(s, N).view(np.uint16)
    Zp = np.arange(G * N // 8, dtype=np.uint32).reshape(G, N // 8).view(np.int32)
    zp = lm.repack_zeros64(Zp, N).view(np.uint32)
    for t in range(N // 16):
        for kb in range(Gk):
            for h in range(2):
                for c in range(16):
                    assert sp[((t * Gk + kb) * 16 + c) * 2 + h] == (2 * kb + h) * N + 16 * t + c
                for w in range(2):
                    assert zp[((t * Gk + kb) * 2 + h) * 2 + w] == (2 * kb + h) * (N // 8) + 2 * t + w


def test_sparse24_model_roundtrip_by_hand():
    # decompress the model's output by hand and compare with the input codes
    from gen import Workload, weights
    w = Workload(cfg=4, M=1, K=256, N=32, sparse24=True)
    d = weights(w)
    vp, meta = lm.sparse24_compress(d["q"], w.K, w.N)
    q = np.full((w.K, w.N), 8, dtype=np.uint8)
    for t in range(w.N // 16):
        for kb in range(w.K // 128):
            for l in range(64):
                n = 16 * t + l % 16
                for h in range(2):
                    word = int(vp[t, kb, l, h])
                    for e in range(8):
                        p = (int(meta[t, kb, l]) >> (16 * h + 2 * e)) & 3
                        k = kb * 128 + 64 * h + 16 * (l // 16) + 4 * (e // 2) + p
                        q[k, n] = (word >> (4 * lm.nib_pos(e))) & 15
    assert np.array_equal(q, d["q"])
    # positions within a run are ascending and distinct
    for h in range(2):
        for g in range(4):
            p0 = (meta >> np.uint32(16 * h + 4 * g)) & np.uint32(3)
            p1 = (meta >> np.uint32(16 * h + 4 * g + 2)) & np.uint32(3)
            assert np.all(p0 < p1)
