"""Pins for the CPU oracle (runs without a GPU).

Each test checks the oracle against something other than itself: hand-derived
fixtures under tests/golden/, exhaustive tables, exact-rational brute force,
closed forms and invariants.  test_planted_mistakes_are_caught plants the
plausible mistakes (dropped term, wrong sign, wrong index, transposed operand)
in copies of the oracle and shows that at least one pin fails for each.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import w4a16_ref as ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---- independent helpers (Python integers only) ------------------------------
def words_from_codes_k(q):
    """Pack [K, N] codes along K with Python integer arithmetic."""
    K, N = q.shape
    out = np.zeros((K // 8, N), dtype=np.int64)
    for i in range(K // 8):
        for n in range(N):
            w = 0
            for j in range(8):
                w += int(q[8 * i + j, n]) * (16 ** j)
            out[i, n] = w
    return out.astype(np.uint32).view(np.int32)


def words_from_codes_n(z):
    G, N = z.shape
    out = np.zeros((G, N // 8), dtype=np.int64)
    for g in range(G):
        for c in range(N // 8):
            w = 0
            for j in range(8):
                w += int(z[g, 8 * c + j]) * (16 ** j)
            out[g, c] = w
    return out.astype(np.uint32).view(np.int32)


def read_fixture(name):
    d = {}
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            d[key] = vals
    return d


# ---- step 1/2: unpack -----------------------------------------------------------
def test_nibble_words_fixture():
    rows = []
    with open(os.path.join(GOLD, "nibble_words.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                parts = line.split()
                rows.append((int(parts[0], 16), [int(v) for v in parts[1:]]))
    Qp = np.array([[w for w, _ in rows]], dtype=np.uint32).view(np.int32)  # [1, N]
    q = oracle.unpack_codes_k(Qp, 8)
    for n, (_, codes) in enumerate(rows):
        assert list(q[:, n]) == codes
    # the same words read as zero-point words (packed along N): codes run along columns
    z = oracle.unpack_codes_n(Qp.reshape(len(rows), 1), 8)
    for g, (_, codes) in enumerate(rows):
        assert list(z[g, :]) == codes


def test_unpack_every_value_every_position():
    # word = v << 4j must give code v at row j and 0 elsewhere, for all v and j
    words = []
    expect = []
    for j in range(8):
        for v in range(16):
            words.append((v << (4 * j)) & 0xFFFFFFFF)
            e = [0] * 8
            e[j] = v
            expect.append(e)
    Qp = np.array([words], dtype=np.uint32).view(np.int32)
    q = oracle.unpack_codes_k(Qp, 8)
    assert np.array_equal(q.T, np.array(expect, dtype=np.uint8))


def test_unpack_all_halfword_patterns():
    p = np.arange(1 << 16, dtype=np.uint32)
    for shift, rows in ((0, range(0, 4)), (16, range(4, 8))):
        Qp = (p << np.uint32(shift)).reshape(1, -1).view(np.int32)
        q = oracle.unpack_codes_k(Qp, 8)
        for j, r in enumerate(rows):
            expect = np.array([(int(x) // (16 ** j)) % 16 for x in p], dtype=np.uint8)
            assert np.array_equal(q[r], expect)
        other = [r for r in range(8) if r not in rows]
        assert not q[other].any()


def test_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(7)
    q = rng.integers(0, 16, size=(64, 24), dtype=np.uint8)
    Qp = words_from_codes_k(q)
    assert np.array_equal(oracle.unpack_codes_k(Qp, 64), q)
    z = rng.integers(0, 16, size=(5, 24), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes_n(words_from_codes_n(z), 24), z)


def test_generator_packing_matches_independent_packer():
    # the shared input generator must produce the canonical format
    from gen import pack_nibbles_along_k, pack_nibbles_along_n
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, size=(32, 16), dtype=np.uint8)
    assert np.array_equal(pack_nibbles_along_k(q), words_from_codes_k(q))
    z = rng.integers(0, 16, size=(3, 16), dtype=np.uint8)
    assert np.array_equal(pack_nibbles_along_n(z), words_from_codes_n(z))


# ---- step 3: dequant ---------------------------------------------------------
SCALES = [1.0, 0.5, 0.002, 0.02, 0.0010004, 2.0 ** -14, 65504.0, 0.0999755859375]


@pytest.mark.parametrize("sv", SCALES)
def test_dequant_exhaustive_closed_form(sv):
    # all 16 x 16 (q, z) pairs, one group of 128 rows x 16 columns, so row k holds q = k % 16
    s16 = np.float16(sv)
    K, N, g = 128, 16, 128
    q = np.array([[k % 16] * N for k in range(K)], dtype=np.uint8)
    z = np.array([list(range(16))], dtype=np.uint8)  # z[0, n] = n
    Qp = words_from_codes_k(q)
    Zp = words_from_codes_n(z)
    s = np.full((1, N), s16, dtype=np.float16)
    W = oracle.dequant(Qp, s, Zp, K, N, g)
    for k in range(K):
        for n in range(N):
            exact = (Fraction(k % 16) - Fraction(n)) * Fraction(float(s16))
            assert Fraction(W[k, n]) == exact
    Wsym = oracle.dequant(Qp, s, None, K, N, g)
    for k in range(16):
        assert Fraction(Wsym[k, 0]) == (Fraction(k) - 8) * Fraction(float(s16))


@pytest.mark.parametrize("g", [64, 128])
def test_dequant_group_indexing(g):
    # scale of group G applies exactly to rows G*g .. G*g+g-1
    K, N = 3 * g, 8
    q = np.full((K, N), 9, dtype=np.uint8)  # q - 8 = 1
    s = np.array([[1.0] * N, [2.0] * N, [4.0] * N], dtype=np.float16)
    W = oracle.dequant(words_from_codes_k(q), s, None, K, N, g)
    assert np.all(W[:g] == 1.0) and np.all(W[g:2 * g] == 2.0) and np.all(W[2 * g:] == 4.0)


def test_dequant_fp16_is_rne_of_exact():
    # (q - z) * s rounded once to fp16; 3 * 0.0999755859375 lies between two fp16 values
    K, N, g = 128, 8, 128
    q = np.full((K, N), 11, dtype=np.uint8)
    s = np.full((1, N), np.float16(0.0999755859375), dtype=np.float16)
    W16 = oracle.dequant_fp16(words_from_codes_k(q), s, None, K, N, g)
    exact = 3 * Fraction(float(np.float16(0.0999755859375)))
    lo = np.float16(float(exact))
    # check it is one of the two neighbours and the nearer one
    cands = [lo, np.nextafter(lo, np.float16(1)), np.nextafter(lo, np.float16(0))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - exact), int(c.view(np.uint16)) & 1))
    assert W16[0, 0] == best


# ---- steps 4-5: products -------------------------------------------------------
@pytest.mark.parametrize("M,K,N,asym,g", [(1, 128, 8, False, 128), (3, 256, 16, True, 128),
                                          (16, 128, 8, True, 128), (2, 256, 8, False, 256),
                                          (3, 256, 16, True, 64), (2, 128, 8, False, 64)])
def test_gemm_vs_exact_rationals(M, K, N, asym, g):
    rng = np.random.default_rng(M * 1000 + K + N)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    Qp = words_from_codes_k(q)
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Zp = words_from_codes_n(rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)) if asym else None
    X = rng.standard_normal((M, K)).astype(np.float16)
    Y = oracle.gemm(X, Qp, s, Zp, g)
    B = oracle.error_bound(X, Qp, s, Zp, g)
    E = oracle.gemm_exact(X, Qp, s, Zp, g)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(Y[m, n]) - E[m][n])
            assert err <= Fraction((K + 2) * 2.0 ** -53) * Fraction(B[m, n])


def test_golden_colsum():
    d = read_fixture("colsum_k128.txt")
    K, N = int(d["K"][0]), int(d["N"][0])
    q = np.array([[(k + n) % 16 for n in range(N)] for k in range(K)], dtype=np.uint8)
    s = np.full((1, N), float(d["s"][0]), dtype=np.float16)
    X = np.ones((1, K), dtype=np.float16)
    Y = oracle.gemm(X, words_from_codes_k(q), s, None, int(d["group"][0]))
    assert np.array_equal(Y[0], np.array([float(v) for v in d["Y"]]))


def test_golden_asym_onehot():
    d = read_fixture("asym_onehot.txt")
    K, N, g = int(d["K"][0]), int(d["N"][0]), int(d["group"][0])
    q = np.array([[15 - n for n in range(N)] for _ in range(K)], dtype=np.uint8)
    Zp = np.array([[0], [int(d["Zp_row1_hex"][0], 16)]], dtype=np.uint32).view(np.int32)
    s = np.array([[1.0] * N, [0.25] * N], dtype=np.float16)
    X = np.zeros((1, K), dtype=np.float16)
    X[0, int(d["onehot_k"][0])] = 1
    Y = oracle.gemm(X, words_from_codes_k(q), s, Zp, g)
    assert np.array_equal(Y[0], np.array([float(v) for v in d["Y"]]))


def test_onehot_rows_select_weight_rows():
    # X = e_k selects row k of W: pins which k and which n every nibble means
    K, N, g = 256, 16, 128
    q = np.array([[(3 * k + 5 * n) % 16 for n in range(N)] for k in range(K)], dtype=np.uint8)
    rng = np.random.default_rng(3)
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    ks = [0, 1, 7, 8, 127, 128, 200, 255]
    X = np.zeros((len(ks), K), dtype=np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1
    Y = oracle.gemm(X, words_from_codes_k(q), s, None, g)
    for m, k in enumerate(ks):
        for n in range(N):
            assert Y[m, n] == ((3 * k + 5 * n) % 16 - 8) * float(s[k // g, n])


def test_integer_matmul_special_case():
    # s = 1, z = 8, one group spanning K: Y = X (Q - 8), an integer matmul
    K, N, M = 256, 16, 4
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, size=(K, N), dtype=np.uint8)
    Xi = rng.integers(-4, 5, size=(M, K))
    Y = oracle.gemm(Xi.astype(np.float16), words_from_codes_k(q), np.ones((1, N), np.float16), None, K)
    assert np.array_equal(Y, (Xi @ (q.astype(np.int64) - 8)).astype(np.float64))


def test_zero_weights_give_exact_zero():
    K, N, M, g = 256, 16, 3, 128
    rng = np.random.default_rng(9)
    X = rng.standard_normal((M, K)).astype(np.float16)
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Y = oracle.gemm(X, words_from_codes_k(np.full((K, N), 8, np.uint8)), s, None, g)
    assert np.all(Y == 0)
    z = rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)
    q = z[np.arange(K) // g, :]
    Y = oracle.gemm(X, words_from_codes_k(q), s, words_from_codes_n(z), g)
    assert np.all(Y == 0)


def test_scale_power_of_two_is_exact():
    K, N, M, g = 512, 16, 5, 128
    rng = np.random.default_rng(13)
    X = rng.standard_normal((M, K)).astype(np.float16)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Y1 = oracle.gemm(X, Qp, s, None, g)
    for j in (1, 3, -2):
        Yj = oracle.gemm(X, Qp, (s.astype(np.float32) * 2.0 ** j).astype(np.float16), None, g)
        assert np.array_equal(Yj, Y1 * 2.0 ** j)


def test_linear_in_x_exact():
    K, N, g = 128, 8, 128
    rng = np.random.default_rng(17)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(1, N)).astype(np.float16)
    X1 = rng.integers(-8, 9, size=(1, K)).astype(np.float16)
    X2 = rng.integers(-8, 9, size=(1, K)).astype(np.float16)
    a, b = 3, -2
    X3 = (a * X1.astype(np.float64) + b * X2.astype(np.float64)).astype(np.float16)
    E1, E2, E3 = (oracle.gemm_exact(X, Qp, s, None, g) for X in (X1, X2, X3))
    for n in range(N):
        assert E3[0][n] == a * E1[0][n] + b * E2[0][n]
    Y1, Y2, Y3 = (oracle.gemm(X, Qp, s, None, g) for X in (X1, X2, X3))
    Bd = oracle.error_bound(X3, Qp, s, None, g)
    assert np.all(np.abs(Y3 - (a * Y1 + b * Y2)) <= 4 * (K + 2) * 2.0 ** -53 * (Bd + 1))


def test_row_permutation():
    K, N, M, g = 256, 16, 6, 128
    rng = np.random.default_rng(19)
    X = rng.standard_normal((M, K)).astype(np.float16)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    P = rng.permutation(M)
    Y = oracle.gemm(X, Qp, s, None, g)
    YP = oracle.gemm(X[P], Qp, s, None, g)
    B = oracle.error_bound(X, Qp, s, None, g)
    assert np.all(np.abs(YP - Y[P]) <= (K + 2) * 2.0 ** -53 * B[P])


def test_sampled_matches_full():
    K, N, M, g = 256, 32, 7, 128
    rng = np.random.default_rng(23)
    X = rng.standard_normal((M, K)).astype(np.float16)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    Zp = words_from_codes_n(rng.integers(0, 16, size=(K // g, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Y = oracle.gemm(X, Qp, s, Zp, g)
    B = oracle.error_bound(X, Qp, s, Zp, g)
    rows, cols = [0, 3, 6], [1, 8, 31, 17]
    Ys, Bs = oracle.gemm_sampled(X, Qp, s, Zp, g, rows, cols)
    assert np.array_equal(Ys, Y[np.ix_(rows, cols)])
    assert np.array_equal(Bs, B[np.ix_(rows, cols)])


# ---- step 6: acceptance ------------------------------------------------------
def _case(M=8, K=1024, N=64, g=128, seed=29):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K)).astype(np.float16)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    return X, Qp, s, g


def test_accept_admits_fp32_accumulation_with_fp16_weights():
    # an implementation that rounds W to fp16, sums in fp32 and rounds Y to fp16
    X, Qp, s, g = _case()
    K, N = X.shape[1], Qp.shape[1]
    W16 = oracle.dequant_fp16(Qp, s, None, K, N, g).astype(np.float32)
    acc = np.zeros((X.shape[0], N), np.float32)
    for k in range(K):  # sequential fp32 accumulation, worst-case-ish order
        acc += X[:, k:k + 1].astype(np.float32) * W16[k:k + 1, :]
    Y = acc.astype(np.float16)
    ok, info = oracle.accept(Y, oracle.gemm(X, Qp, s, None, g), oracle.error_bound(X, Qp, s, None, g))
    assert ok, info


def test_accept_rejects_wrong_results():
    X, Qp, s, g = _case()
    Yref = oracle.gemm(X, Qp, s, None, g)
    B = oracle.error_bound(X, Qp, s, None, g)
    Y = Yref.astype(np.float16)
    assert oracle.accept(Y, Yref, B)[0]
    bad = Y.copy()
    bad[3, 5] = np.float16(float(bad[3, 5]) + 0.05 * float(B[3, 5]) + 0.01)
    assert not oracle.accept(bad, Yref, B)[0]
    nan = Y.copy()
    nan[0, 0] = np.nan
    assert not oracle.accept(nan, Yref, B)[0]
    # dropping the last group is a 1/8 relative error: rejected
    K = X.shape[1]
    Xt = X.copy()
    Xt[:, K - g:] = 0
    assert not oracle.accept(oracle.gemm(Xt, Qp, s, None, g).astype(np.float16), Yref, B)[0]


def test_check_24():
    K, N = 128, 8
    q = np.full((K, N), 8, np.uint8)
    q[0, :] = 3
    q[1, :] = 15  # 2 nonzero in the first run
    assert oracle.check_24(words_from_codes_k(q), K)
    q[2, 4] = 1  # 3 nonzero in the run of column 4
    assert not oracle.check_24(words_from_codes_k(q), K)


def test_generator_24_structure_and_distribution():
    from gen import Workload, weights
    w = Workload(cfg=4, M=16, K=256, N=64, sparse24=True)
    d = weights(w)
    assert oracle.check_24(d["Qp"], w.K)
    keep = d["keep"].reshape(w.K // 4, 4, w.N)
    assert np.all(keep.sum(axis=1) == 2)
    assert np.all(d["q"][~d["keep"]] == 8)


# ---- planted mistakes --------------------------------------------------------
def _pins_pass(mod):
    """Run a subset of the pins above against a (possibly mutated) oracle module."""
    checks = []
    # one-hot selection
    K, N, g = 256, 16, 128
    q = np.array([[(3 * k + 5 * n) % 16 for n in range(N)] for k in range(K)], dtype=np.uint8)
    s = np.random.default_rng(3).uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    X = np.zeros((3, K), dtype=np.float16)
    ks = [1, 130, 255]
    for m, k in enumerate(ks):
        X[m, k] = 1
    Y = mod.gemm(X, words_from_codes_k(q), s, None, g)
    checks.append(all(Y[m, n] == ((3 * k + 5 * n) % 16 - 8) * float(s[k // g, n])
                      for m, k in enumerate(ks) for n in range(N)))
    # asym golden
    d = read_fixture("asym_onehot.txt")
    K2, N2 = int(d["K"][0]), int(d["N"][0])
    q2 = np.array([[15 - n for n in range(N2)] for _ in range(K2)], dtype=np.uint8)
    Zp = np.array([[0], [0x76543210]], dtype=np.uint32).view(np.int32)
    s2 = np.array([[1.0] * N2, [0.25] * N2], dtype=np.float16)
    X2 = np.zeros((1, K2), dtype=np.float16)
    X2[0, 130] = 1
    Y2 = mod.gemm(X2, words_from_codes_k(q2), s2, Zp, 128)
    checks.append(np.array_equal(Y2[0], np.array([float(v) for v in d["Y"]])))
    # non-square tiny brute force
    rng = np.random.default_rng(31)
    M3, K3, N3 = 2, 256, 8
    X3 = rng.standard_normal((M3, K3)).astype(np.float16)
    Qp3 = words_from_codes_k(rng.integers(0, 16, size=(K3, N3), dtype=np.uint8))
    s3 = rng.uniform(0.002, 0.02, size=(2, N3)).astype(np.float16)
    Y3 = mod.gemm(X3, Qp3, s3, None, 128)
    E3 = oracle.gemm_exact(X3, Qp3, s3, None, 128)
    checks.append(all(abs(Fraction(Y3[m, n]) - E3[m][n]) < Fraction(1, 10 ** 9)
                      for m in range(M3) for n in range(N3)))
    return all(checks)


def test_planted_mistakes_are_caught(monkeypatch):
    import types
    assert _pins_pass(ref)

    def mutant(**overrides):
        m = types.ModuleType("mutant")
        m.__dict__.update({k: getattr(ref, k) for k in dir(ref) if not k.startswith("__")})
        m.__dict__.update(overrides)
        # rebind the functions so that they see the overrides
        for name in ("dequant", "gemm"):
            f = getattr(ref, name)
            if name not in overrides:
                m.__dict__[name] = types.FunctionType(f.__code__, m.__dict__, name, f.__defaults__)
        return m

    def unpack_msb_first(Qp, K, cols=None):
        U = np.ascontiguousarray(Qp).view(np.uint32)
        if cols is not None:
            U = U[:, np.asarray(cols)]
        q = np.empty((K, U.shape[1]), dtype=np.uint8)
        for k in range(8):
            q[k::8] = ((U >> np.uint32(4 * (7 - k))) & np.uint32(15)).astype(np.uint8)
        return q

    def unpack_signed(Qp, K, cols=None):  # arithmetic shift on int32: wrong high nibble handling
        U = np.ascontiguousarray(Qp).view(np.int32).astype(np.int64)
        if cols is not None:
            U = U[:, np.asarray(cols)]
        q = np.empty((K, U.shape[1]), dtype=np.uint8)
        for k in range(8):
            q[k::8] = ((U >> (4 * k)) & (15 if k < 7 else 7)).astype(np.uint8)
        return q

    def zero_points_sign(G, N, Zp):
        z = ref.zero_points(G, N, Zp)
        return (16 - z.astype(np.int64)).astype(np.uint8) % 16

    def zero_points_transposed(G, N, Zp):
        if Zp is None:
            return np.full((G, N), 8, dtype=np.uint8)
        z = ref.unpack_codes_n(Zp, N)
        return z[::-1].copy()

    def dequant_drop_zero(Qp, s, Zp, K, N, group, cols=None):
        q = ref.unpack_codes_k(Qp, K, cols).astype(np.float64)
        s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
        if cols is not None:
            s64 = s64[:, np.asarray(cols)]
        return q * s64[np.arange(K) // group, :]

    def dequant_wrong_group(Qp, s, Zp, K, N, group, cols=None):
        q = ref.unpack_codes_k(Qp, K, cols).astype(np.float64)
        z = ref.zero_points(K // group, N, Zp).astype(np.float64)
        s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
        r = np.minimum(np.arange(K) // (group * 2), K // group - 1)
        return (q - z[r, :]) * s64[r, :]

    def gemm_transposed_operand(X, Qp, s, Zp, group, rows_per_chunk=1024):
        K = X.shape[1]
        N = Qp.shape[1]
        W = ref.dequant(Qp, s, Zp, K, N, group)
        W = W.reshape(N, K).T if W.shape[0] == W.shape[1] else W[::-1]
        return X.astype(np.float64) @ W

    mutants = [
        mutant(unpack_codes_k=unpack_msb_first),
        mutant(unpack_codes_k=unpack_signed),
        mutant(zero_points=zero_points_sign),
        mutant(zero_points=zero_points_transposed),
        mutant(dequant=dequant_drop_zero),
        mutant(dequant=dequant_wrong_group),
        mutant(gemm=gemm_transposed_operand),
    ]
    for i, m in enumerate(mutants):
        assert not _pins_pass(m), f"mutant {i} survived the pins"


# ---- W4A8: fp8 (E4M3) activations --------------------------------------------------
def _e4m3_fixture():
    out = []
    with open(os.path.join(GOLD, "e4m3_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                out.append((int(code, 16), float(val)))
    return out


def _torch_e4m3(codes):
    import torch
    c = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_golden_fixture():
    for code, val in _e4m3_fixture():
        v = float(oracle.decode_e4m3(np.array([code], np.uint8))[0])
        if np.isnan(val):
            assert np.isnan(v), hex(code)
        else:
            assert v == val and np.signbit(v) == np.signbit(val), hex(code)


def test_e4m3_exhaustive_vs_library():
    # every byte code against torch's float8_e4m3fn (a library decode of the same format)
    c = np.arange(256, dtype=np.uint8)
    assert np.array_equal(oracle.decode_e4m3(c), _torch_e4m3(c), equal_nan=True)


def _w4a8_exact(X8, a, Qp, s, Zp, g):
    """sum_k a[m] x[m,k] (q - z) s in exact rationals; x from the library decode,
    codes read bit by bit from Python integers."""
    M, K = X8.shape
    N = Qp.shape[1]
    xv = _torch_e4m3(X8)
    Qw = [[int(v) & 0xFFFFFFFF for v in row] for row in np.asarray(Qp, dtype=np.int64)]
    Zw = None if Zp is None else [[int(v) & 0xFFFFFFFF for v in row] for row in np.asarray(Zp, dtype=np.int64)]
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        am = Fraction(1) if a is None else Fraction(float(np.float32(a[m])))
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                q = (Qw[k // 8][n] >> (4 * (k % 8))) % 16
                z = 8 if Zw is None else (Zw[k // g][n // 8] >> (4 * (n % 8))) % 16
                acc += Fraction(float(xv[m, k])) * (q - z) * Fraction(float(s[k // g, n]))
            out[m][n] = am * acc
    return out


def _random_e4m3(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((c & 0x7F) == 0x7F, np.uint8(0x38), c).astype(np.uint8)  # no NaN codes


@pytest.mark.parametrize("M,K,N,asym,scaled", [(1, 128, 8, False, False), (3, 256, 16, True, True),
                                               (4, 128, 8, True, False), (2, 256, 8, False, True)])
def test_w4a8_gemm_vs_exact_rationals(M, K, N, asym, scaled):
    rng = np.random.default_rng(7 * M + K + N)
    g = 128
    X8 = _random_e4m3(rng, (M, K))
    a = rng.uniform(0.001, 0.01, size=M).astype(np.float32) if scaled else None
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Zp = words_from_codes_n(rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)) if asym else None
    Y = oracle.gemm_w4a8(X8, a, Qp, s, Zp, g)
    B = oracle.error_bound_w4a8(X8, a, Qp, s, Zp, g)
    E = _w4a8_exact(X8, a, Qp, s, Zp, g)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(Y[m, n]) - E[m][n]) <= Fraction((K + 2) * 2.0 ** -53) * Fraction(B[m, n])


def test_w4a8_onehot_rows_and_row_scale():
    # x8 = 1.0 (code 0x38) at k, a = 2^j: row m of Y is exactly 2^j * W[k, :]
    K, N, g = 256, 16, 128
    q = np.array([[(5 * k + 3 * n) % 16 for n in range(N)] for k in range(K)], dtype=np.uint8)
    s = np.random.default_rng(4).uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    ks = [0, 9, 127, 128, 255]
    X8 = np.zeros((len(ks), K), dtype=np.uint8)
    for m, k in enumerate(ks):
        X8[m, k] = 0x38
    a = np.array([1.0, 2.0, 0.5, 4.0, 0.25], dtype=np.float32)
    Y = oracle.gemm_w4a8(X8, a, words_from_codes_k(q), s, None, g)
    for m, k in enumerate(ks):
        for n in range(N):
            assert Y[m, n] == float(a[m]) * ((5 * k + 3 * n) % 16 - 8) * float(s[k // g, n])


def test_w4a8_row_scale_is_per_row_and_exact():
    rng = np.random.default_rng(21)
    M, K, N, g = 5, 256, 16, 128
    X8 = _random_e4m3(rng, (M, K))
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Y1 = oracle.gemm_w4a8(X8, None, Qp, s, None, g)
    assert np.array_equal(Y1, oracle.gemm_w4a8(X8, np.ones(M, np.float32), Qp, s, None, g))
    p = np.array([2.0, 0.5, 8.0, 1.0, 0.125], dtype=np.float32)
    assert np.array_equal(oracle.gemm_w4a8(X8, p, Qp, s, None, g), Y1 * p[:, None].astype(np.float64))


def _pins_w4a8_pass(mod):
    checks = []
    for code, val in _e4m3_fixture():
        v = float(mod.decode_e4m3(np.array([code], np.uint8))[0])
        checks.append(np.isnan(v) if np.isnan(val) else v == val)
    rng = np.random.default_rng(5)
    M, K, N = 3, 256, 8
    X8 = _random_e4m3(rng, (M, K))
    a = np.array([0.5, 0.003, 7.0], dtype=np.float32)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // 128, N)).astype(np.float16)
    Y = mod.gemm_w4a8(X8, a, Qp, s, None, 128)
    E = _w4a8_exact(X8, a, Qp, s, None, 128)
    checks.append(all(abs(Fraction(Y[m, n]) - E[m][n]) < Fraction(1, 10 ** 9)
                      for m in range(M) for n in range(N)))
    return all(checks)


def test_w4a8_planted_mistakes_are_caught():
    import types
    assert _pins_w4a8_pass(ref)

    def mutant(**overrides):
        m = types.ModuleType("mutant")
        m.__dict__.update({k: getattr(ref, k) for k in dir(ref) if not k.startswith("__")})
        m.__dict__.update(overrides)
        for name in ("activations_w4a8", "gemm_w4a8"):
            if name not in overrides:
                f = getattr(ref, name)
                m.__dict__[name] = types.FunctionType(f.__code__, m.__dict__, name, f.__defaults__)
        return m

    def decode_bias8(codes):  # exponent bias 8 (the other FP8 E4M3 convention)
        return ref.decode_e4m3(codes) / 2.0

    def decode_no_subnormal(codes):  # e = 0 read as a normal number
        c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
        v = ref.decode_e4m3(c)
        e0 = ((c >> 3) & 15) == 0
        mag = np.ldexp(1.0 + (c & 7) / 8.0, -7)
        return np.where(e0 & ((c & 7) != 0), np.where(c >> 7, -mag, mag), v)

    def decode_no_sign(codes):
        return np.abs(ref.decode_e4m3(codes))

    def acts_scale_by_column(X8, xscale):  # row scale applied along K instead of M
        Xv = ref.decode_e4m3(X8)
        if xscale is not None:
            sc = np.resize(np.asarray(xscale, np.float64), Xv.shape[1])
            Xv = Xv * sc[None, :]
        return Xv

    def acts_scale_dropped(X8, xscale):
        return ref.decode_e4m3(X8)

    mutants = [
        mutant(decode_e4m3=decode_bias8),
        mutant(decode_e4m3=decode_no_subnormal),
        mutant(decode_e4m3=decode_no_sign),
        mutant(activations_w4a8=acts_scale_by_column),
        mutant(activations_w4a8=acts_scale_dropped),
    ]
    for i, m in enumerate(mutants):
        assert not _pins_w4a8_pass(m), f"W4A8 mutant {i} survived the pins"


def test_generator_fp8_activations():
    from gen import Workload, activations_fp8
    w = Workload(cfg=1, M=5, K=256, N=64)
    codes, a = activations_fp8(w)
    v = oracle.decode_e4m3(codes)
    assert codes.dtype == np.uint8 and a.dtype == np.float32 and not np.isnan(v).any()
    # every row uses the full E4M3 range: its largest magnitude is 448
    assert np.all(np.abs(v).max(axis=1) == 448.0)


# ---- MXFP4 weights (block scales applied inside the matrix instruction) ---------
def _e2m1_fixture():
    out = []
    with open(os.path.join(GOLD, "e2m1_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                out.append((int(code, 16), float(val)))
    return out


def test_e2m1_golden_fixture_is_every_code():
    fx = _e2m1_fixture()
    assert sorted(c for c, _ in fx) == list(range(16))
    for code, val in fx:
        v = float(oracle.decode_e2m1(np.array([code]))[0])
        assert v == val and np.signbit(v) == np.signbit(val), code


def test_e8m0_vs_library():
    # every scale byte against torch's float8_e8m0fnu (a library decode of the format)
    import torch
    c = np.arange(256, dtype=np.uint8)
    lib = torch.from_numpy(c).view(torch.float8_e8m0fnu).float().double().numpy()
    assert np.array_equal(oracle.decode_e8m0(c), lib, equal_nan=True)
    assert oracle.decode_e8m0(np.array([127], np.uint8))[0] == 1.0


def _mx_exact(X8, a, Qp, E):
    """Brute force in exact rationals with Python integers: unpack nibble k % 8 of word
    k // 8, E2M1 from its bit fields, the block scale 2^(E[k // 32] - 127)."""
    M, K = X8.shape
    N = Qp.shape[1]
    fx = dict(_e2m1_fixture())
    e4 = dict(_e4m3_exact_table())
    out = []
    for m in range(M):
        row = []
        am = Fraction(float(a[m])) if a is not None else Fraction(1)
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                code = (int(Qp[k // 8, n]) & 0xFFFFFFFF) >> (4 * (k % 8)) & 15
                e = int(E[k // 32, n]) - 127
                sc = Fraction(2) ** e
                acc += e4[int(X8[m, k])] * Fraction(fx[code]) * sc
            row.append(am * acc)
        out.append(row)
    return out


def _e4m3_exact_table():
    # exact values of every finite E4M3 code from its bit fields (no float arithmetic)
    t = []
    for c in range(256):
        s, e, mm = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and mm == 7:
            continue
        v = Fraction(mm, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(mm, 8)) * Fraction(2) ** (e - 7)
        t.append((c, -v if s else v))
    return t


@pytest.mark.parametrize("M,K,N,scaled", [(1, 64, 8, False), (3, 128, 8, True), (2, 96, 16, True)])
def test_mxfp4_gemm_vs_exact_rationals(M, K, N, scaled):
    rng = np.random.default_rng(11 * M + K + N)
    X8 = _random_e4m3(rng, (M, K))
    a = rng.uniform(0.001, 0.01, size=M).astype(np.float32) if scaled else None
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    E = rng.integers(110, 140, size=(K // 32, N), dtype=np.uint8)
    Y = oracle.gemm_mxfp4(X8, a, Qp, E)
    B = oracle.error_bound_mxfp4(X8, a, Qp, E)
    Ex = _mx_exact(X8, a, Qp, E)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(Y[m, n]) - Ex[m][n]) <= Fraction((K + 2) * 2.0 ** -53) * Fraction(B[m, n])


def test_mxfp4_onehot_rows_select_scaled_codes():
    # x8 = 1.0 at row k: row m of Y is e2m1(q[k, n]) * 2^(E[k // 32, n] - 127) exactly;
    # rows on both sides of every 32-row boundary pin the block index
    K, N = 128, 16
    q = np.array([[(3 * k + 5 * n) % 16 for n in range(N)] for k in range(K)], dtype=np.uint8)
    E = np.array([[120 + (b + n) % 7 for n in range(N)] for b in range(K // 32)], dtype=np.uint8)
    ks = [0, 1, 31, 32, 33, 63, 64, 95, 96, 127]
    X8 = np.zeros((len(ks), K), dtype=np.uint8)
    for m, k in enumerate(ks):
        X8[m, k] = 0x38
    fx = dict(_e2m1_fixture())
    Y = oracle.gemm_mxfp4(X8, None, words_from_codes_k(q), E)
    for m, k in enumerate(ks):
        for n in range(N):
            assert Y[m, n] == fx[(3 * k + 5 * n) % 16] * 2.0 ** (int(E[k // 32, n]) - 127)


def test_mxfp4_unit_scales_reduce_to_an_integer_product():
    # with every block scale 2^0 and codes restricted to the integer values {0, 1, 2,
    # 3, 4, 6} (and negatives), Y is an integer matrix product (exact in int64)
    rng = np.random.default_rng(8)
    M, K, N = 4, 256, 24
    ints = {2: 1, 4: 2, 5: 3, 6: 4, 7: 6, 10: -1, 12: -2, 13: -3, 14: -4, 15: -6, 0: 0}
    codes = np.array(list(ints.keys()), dtype=np.uint8)
    q = rng.choice(codes, size=(K, N))
    Wi = np.vectorize(ints.get)(q).astype(np.int64)
    Xi = rng.integers(-8, 9, size=(M, K))
    X8 = np.array([[dict((int(v), c) for c, v in _e4m3_exact_table() if v.denominator == 1
                          and -8 <= v <= 8 and not (v == 0 and c == 0x80))[int(x)] for x in r]
                   for r in Xi], dtype=np.uint8)
    E = np.full((K // 32, N), 127, dtype=np.uint8)
    Y = oracle.gemm_mxfp4(X8, None, words_from_codes_k(q), E)
    assert np.array_equal(Y, (Xi @ Wi).astype(np.float64))


def _pins_mx_pass(mod):
    checks = []
    for code, val in _e2m1_fixture():
        checks.append(float(mod.decode_e2m1(np.array([code]))[0]) == val)
    rng = np.random.default_rng(9)
    M, K, N = 2, 128, 8
    X8 = _random_e4m3(rng, (M, K))
    a = np.array([0.5, 0.003], dtype=np.float32)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    E = rng.integers(115, 135, size=(K // 32, N), dtype=np.uint8)
    Y = mod.gemm_mxfp4(X8, a, Qp, E)
    Ex = _mx_exact(X8, a, Qp, E)
    checks.append(all(abs(Fraction(Y[m, n]) - Ex[m][n]) < Fraction(1, 10 ** 9)
                      for m in range(M) for n in range(N)))
    return all(checks)


def test_mxfp4_planted_mistakes_are_caught():
    import types
    assert _pins_mx_pass(ref)

    def mutant(**overrides):
        m = types.ModuleType("mutant")
        m.__dict__.update({k: getattr(ref, k) for k in dir(ref) if not k.startswith("__")})
        m.__dict__.update(overrides)
        for name in ("dequant_mxfp4", "gemm_mxfp4"):
            if name not in overrides:
                f = getattr(ref, name)
                m.__dict__[name] = types.FunctionType(f.__code__, m.__dict__, name, f.__defaults__)
        return m

    def e2m1_bias0(codes):  # exponent bias 0 instead of 1
        return ref.decode_e2m1(codes) * 2.0

    def e2m1_no_subnormal(codes):  # e = 0 read as 2^-1 * (1 + m/2)
        c = np.asarray(codes).astype(np.int64) & 15
        v = ref.decode_e2m1(c)
        e0 = ((c >> 1) & 3) == 0
        mag = 0.5 * (1 + (c & 1) / 2.0)
        return np.where(e0, np.where(c >> 3, -mag, mag), v)

    def e8m0_bias128(codes):
        return ref.decode_e8m0(codes) / 2.0

    def dq_block16(Qp, E, K, N, cols=None):  # the scale block read as 16 rows
        q = ref.unpack_codes_k(Qp, K, cols)
        Ec = E if cols is None else E[:, np.asarray(cols)]
        sc = np.repeat(ref.decode_e8m0(Ec), 16, axis=0)
        sc = np.concatenate([sc, sc])[:K]
        return ref.decode_e2m1(q) * sc

    def dq_nibbles_swapped(Qp, E, K, N, cols=None):  # high nibble of each byte first
        q = ref.unpack_codes_k(Qp, K, cols)
        q = q.reshape(K // 2, 2, -1)[:, ::-1, :].reshape(K, -1)
        Ec = E if cols is None else E[:, np.asarray(cols)]
        return ref.decode_e2m1(q) * np.repeat(ref.decode_e8m0(Ec), 32, axis=0)

    mutants = [
        mutant(decode_e2m1=e2m1_bias0),
        mutant(decode_e2m1=e2m1_no_subnormal),
        mutant(decode_e8m0=e8m0_bias128),
        mutant(dequant_mxfp4=dq_block16),
        mutant(dequant_mxfp4=dq_nibbles_swapped),
    ]
    for i, m in enumerate(mutants):
        assert not _pins_mx_pass(m), f"MXFP4 mutant {i} survived the pins"


def test_generator_mxfp4_weights():
    from gen import Workload, weights_mxfp4
    d = weights_mxfp4(Workload(cfg=9, M=1, K=256, N=32), seed=3)
    assert d["Qp"].shape == (32, 32) and d["E"].shape == (8, 32)
    assert d["E"].min() >= 119 and d["E"].max() <= 124
    assert np.array_equal(ref.unpack_codes_k(d["Qp"], 256), d["q"])
    assert len(np.unique(d["q"])) == 16


def test_mxfp4_sampled_equals_full_at_the_samples():
    # the full-size GPU tests compare against the sampled oracle: it must be the full one
    # restricted to the sampled rows and columns (row scales follow their rows)
    rng = np.random.default_rng(31)
    M, K, N = 7, 256, 48
    X8 = _random_e4m3(rng, (M, K))
    a = rng.uniform(0.001, 0.01, size=M).astype(np.float32)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    E = rng.integers(115, 135, size=(K // 32, N), dtype=np.uint8)
    rows, cols = [0, 3, 6], [1, 17, 32, 47]
    Y, B = oracle.gemm_mxfp4_sampled(X8, a, Qp, E, rows, cols)
    # equal up to the fp64 rounding of a different summation order inside the library matmul
    Bf = oracle.error_bound_mxfp4(X8, a, Qp, E)[np.ix_(rows, cols)]
    assert np.all(np.abs(Y - oracle.gemm_mxfp4(X8, a, Qp, E)[np.ix_(rows, cols)]) <= 1e-12 * Bf)
    assert np.allclose(B, Bf, rtol=1e-12, atol=0)


# ---- the tolerance scale Bnd = sum_k |X[m,k] * W[k,n]| --------------------------
# Every per-element acceptance limit in the GPU tests is 5e-3 * Bnd + 1e-4, so the
# bound functions are pinned against an exact-rational sum built here from the bit
# fields with Python integers (no NumPy unpacking, no matrix product), and planted
# mistakes in them (abs dropped, a constant factor, fp16-rounded weights with slack,
# a dropped scale) must each fail.
def _exact_abs_sum(xvals, Qp, wval):
    """[[sum_k |x[m][k]| * |w(k, n)|]] in Fractions; x as Fractions, w(k, n) a callable
    returning the exact weight of row k, column n."""
    M, K = len(xvals), len(xvals[0])
    N = Qp.shape[1]
    return [[sum((abs(xvals[m][k]) * abs(wval(k, n)) for k in range(K)), Fraction(0))
             for n in range(N)] for m in range(M)]


def _int4_weight(Qp, s, Zp, g):
    Qw = [[int(v) & 0xFFFFFFFF for v in row] for row in np.asarray(Qp, dtype=np.int64)]
    Zw = None if Zp is None else [[int(v) & 0xFFFFFFFF for v in row]
                                  for row in np.asarray(Zp, dtype=np.int64)]
    Sf = [[Fraction(float(v)) for v in row] for row in np.asarray(s, dtype=np.float16)]

    def w(k, n):
        q = (Qw[k // 8][n] >> (4 * (k % 8))) % 16
        z = 8 if Zw is None else (Zw[k // g][n // 8] >> (4 * (n % 8))) % 16
        return (q - z) * Sf[k // g][n]
    return w


def _mx_weight(Qp, E):
    fx = dict(_e2m1_fixture())

    def w(k, n):
        code = ((int(Qp[k // 8, n]) & 0xFFFFFFFF) >> (4 * (k % 8))) & 15
        return Fraction(fx[code]) * Fraction(2) ** (int(E[k // 32, n]) - 127)
    return w


def _e4m3_rows(X8, a):
    """Exact activation values a[m] * x8[m, k] from the bit-field table."""
    e4 = dict(_e4m3_exact_table())
    return [[(Fraction(1) if a is None else Fraction(float(np.float32(a[m])))) * e4[int(c)]
             for c in row] for m, row in enumerate(np.asarray(X8))]


def _bound_close(B, exact, K):
    """B (fp64) equals the exact positive sum up to the fp64 rounding of K additions."""
    B = np.asarray(B)
    for m in range(B.shape[0]):
        for n in range(B.shape[1]):
            e = exact[m][n]
            if abs(Fraction(float(B[m, n])) - e) > Fraction((K + 2) * 2.0 ** -53) * e:
                return False
    return True


def _bound_cases():
    rng = np.random.default_rng(77)
    cases = []
    for (M, K, N, asym, g) in [(2, 256, 8, False, 128), (3, 256, 16, True, 128),
                               (2, 128, 8, True, 64), (2, 512, 8, True, 256)]:
        X = rng.standard_normal((M, K)).astype(np.float16)
        Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
        s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
        Zp = words_from_codes_n(rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)) if asym else None
        cases.append((X, Qp, s, Zp, g))
    return cases


def _pins_bounds_pass(mod):
    checks = []
    # W4A16: full bound and the sampled one, sym / asym, groups of 64, 128, 256
    for X, Qp, s, Zp, g in _bound_cases():
        M, K = X.shape
        N = Qp.shape[1]
        xv = [[Fraction(float(v)) for v in row] for row in X]
        ex = _exact_abs_sum(xv, Qp, _int4_weight(Qp, s, Zp, g))
        checks.append(_bound_close(mod.error_bound(X, Qp, s, Zp, g), ex, K))
        rows, cols = [M - 1, 0], [N - 1, 2, 5]
        _, Bs = mod.gemm_sampled(X, Qp, s, Zp, g, rows, cols)
        checks.append(_bound_close(Bs, [[ex[r][c] for c in cols] for r in rows], K))
    # W4A8: fp32 row scales (or none), sym / asym, full and sampled
    rng = np.random.default_rng(78)
    for (M, K, N, asym, scaled) in [(3, 256, 8, True, True), (2, 128, 16, False, False),
                                    (3, 128, 8, False, True)]:
        g = 128
        X8 = _random_e4m3(rng, (M, K))
        a = np.array([0.5, 0.0039, 7.25][:M], dtype=np.float32) if scaled else None
        Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
        s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
        Zp = words_from_codes_n(rng.integers(0, 16, size=(K // g, N), dtype=np.uint8)) if asym else None
        xv = _e4m3_rows(X8, a)
        ex = _exact_abs_sum(xv, Qp, _int4_weight(Qp, s, Zp, g))
        checks.append(_bound_close(mod.error_bound_w4a8(X8, a, Qp, s, Zp, g), ex, K))
        rows, cols = [M - 1, 0], [N - 1, 3]
        Ys, Bs = mod.gemm_w4a8_sampled(X8, a, Qp, s, Zp, g, rows, cols)
        checks.append(_bound_close(Bs, [[ex[r][c] for c in cols] for r in rows], K))
        ey = _w4a8_exact(X8, a, Qp, s, Zp, g)
        checks.append(all(abs(Fraction(float(Ys[i, j])) - ey[r][c])
                          <= Fraction((K + 2) * 2.0 ** -53) * ex[r][c]
                          for i, r in enumerate(rows) for j, c in enumerate(cols)))
    # MXFP4: E8M0 block scales and row scales, full and sampled
    for (M, K, N, scaled) in [(2, 128, 8, True), (3, 64, 16, False)]:
        X8 = _random_e4m3(rng, (M, K))
        a = np.array([0.75, 0.0061, 3.0][:M], dtype=np.float32) if scaled else None
        Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
        E = rng.integers(110, 140, size=(K // 32, N), dtype=np.uint8)
        ex = _exact_abs_sum(_e4m3_rows(X8, a), Qp, _mx_weight(Qp, E))
        checks.append(_bound_close(mod.error_bound_mxfp4(X8, a, Qp, E), ex, K))
        rows, cols = [M - 1, 0], [N - 1, 1]
        _, Bs = mod.gemm_mxfp4_sampled(X8, a, Qp, E, rows, cols)
        checks.append(_bound_close(Bs, [[ex[r][c] for c in cols] for r in rows], K))
    return all(checks)


def test_error_bounds_equal_exact_rational_sums():
    assert _pins_bounds_pass(ref)


def test_w4a8_sampled_matches_full_at_the_samples():
    # the full-size W4A8 GPU tests compare against the sampled oracle
    rng = np.random.default_rng(32)
    M, K, N, g = 6, 256, 40, 128
    X8 = _random_e4m3(rng, (M, K))
    a = rng.uniform(0.001, 0.01, size=M).astype(np.float32)
    Qp = words_from_codes_k(rng.integers(0, 16, size=(K, N), dtype=np.uint8))
    s = rng.uniform(0.002, 0.02, size=(K // g, N)).astype(np.float16)
    Zp = words_from_codes_n(rng.integers(0, 16, size=(K // g, N), dtype=np.uint8))
    rows, cols = [5, 0, 3], [39, 8, 1, 16]
    Y, B = oracle.gemm_w4a8_sampled(X8, a, Qp, s, Zp, g, rows, cols)
    Bf = oracle.error_bound_w4a8(X8, a, Qp, s, Zp, g)[np.ix_(rows, cols)]
    assert np.all(np.abs(Y - oracle.gemm_w4a8(X8, a, Qp, s, Zp, g)[np.ix_(rows, cols)]) <= 1e-12 * Bf)
    assert np.allclose(B, Bf, rtol=1e-12, atol=0)


def test_bound_planted_mistakes_are_caught():
    import types

    def mutant(**overrides):
        m = types.ModuleType("mutant")
        m.__dict__.update({k: getattr(ref, k) for k in dir(ref) if not k.startswith("__")})
        m.__dict__.update(overrides)
        return m

    def eb_abs_dropped_on_w(X, Qp, s, Zp, group, rows_per_chunk=1024):
        K, N = X.shape[1], Qp.shape[1]
        return np.abs(X.astype(np.float64)) @ ref.dequant(Qp, s, Zp, K, N, group)

    def eb_times_10(X, Qp, s, Zp, group, rows_per_chunk=1024):
        return 10.0 * ref.error_bound(X, Qp, s, Zp, group)

    def eb_fp16_weights_slack(X, Qp, s, Zp, group, rows_per_chunk=1024):
        K, N = X.shape[1], Qp.shape[1]
        W16 = ref.dequant_fp16(Qp, s, Zp, K, N, group).astype(np.float64)
        return 2.0 * (np.abs(X.astype(np.float64)) @ np.abs(W16))

    def eb_abs_of_sum(X, Qp, s, Zp, group, rows_per_chunk=1024):
        return np.abs(ref.gemm(X, Qp, s, Zp, group))

    def eb_scale_dropped(X, Qp, s, Zp, group, rows_per_chunk=1024):
        return ref.error_bound(X, Qp, np.ones_like(s), Zp, group)

    def sampled_abs_dropped_on_x(X, Qp, s, Zp, group, rows, cols):
        K, N = X.shape[1], Qp.shape[1]
        W = ref.dequant(Qp, s, Zp, K, N, group, cols=cols)
        Xr = X[np.asarray(rows)].astype(np.float64)
        return Xr @ W, Xr @ np.abs(W)

    def w8_row_scale_dropped(X8, xscale, Qp, s, Zp, group):
        return ref.error_bound_w4a8(X8, None, Qp, s, Zp, group)

    def w8_times_10(X8, xscale, Qp, s, Zp, group):
        return 10.0 * ref.error_bound_w4a8(X8, xscale, Qp, s, Zp, group)

    def w8_sampled_row_scale_unsliced(X8, xscale, Qp, s, Zp, group, rows, cols):
        K, N = X8.shape[1], Qp.shape[1]
        W = ref.dequant(Qp, s, Zp, K, N, group, cols=cols)
        r = np.asarray(rows)
        a = None if xscale is None else np.asarray(xscale)[:len(r)]
        Xr = ref.activations_w4a8(X8[r], a)
        return Xr @ W, np.abs(Xr) @ np.abs(W)

    def mx_times_10(X8, xscale, Qp, E):
        return 10.0 * ref.error_bound_mxfp4(X8, xscale, Qp, E)

    def mx_block_scale_dropped(X8, xscale, Qp, E):
        return ref.error_bound_mxfp4(X8, xscale, Qp, np.full_like(E, 127))

    def mx_sampled_abs_dropped(X8, xscale, Qp, E, rows, cols):
        K, N = X8.shape[1], Qp.shape[1]
        W = ref.dequant_mxfp4(Qp, E, K, N, cols=cols)
        r = np.asarray(rows)
        Xr = ref.activations_w4a8(X8[r], None if xscale is None else np.asarray(xscale)[r])
        return Xr @ W, np.abs(Xr @ W)

    mutants = [
        mutant(error_bound=eb_abs_dropped_on_w),
        mutant(error_bound=eb_times_10),
        mutant(error_bound=eb_fp16_weights_slack),
        mutant(error_bound=eb_abs_of_sum),
        mutant(error_bound=eb_scale_dropped),
        mutant(gemm_sampled=sampled_abs_dropped_on_x),
        mutant(error_bound_w4a8=w8_row_scale_dropped),
        mutant(error_bound_w4a8=w8_times_10),
        mutant(gemm_w4a8_sampled=w8_sampled_row_scale_unsliced),
        mutant(error_bound_mxfp4=mx_times_10),
        mutant(error_bound_mxfp4=mx_block_scale_dropped),
        mutant(gemm_mxfp4_sampled=mx_sampled_abs_dropped),
    ]
    for i, m in enumerate(mutants):
        assert not _pins_bounds_pass(m), f"bound mutant {i} survived the pins"
