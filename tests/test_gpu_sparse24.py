"""GPU parity of the 2:4-structured-sparse path (compress, decompress, smfmac GEMM)
against the CPU oracle.  The oracle of a 2:4 weight is the dense oracle on the
pruned codes (pruned positions carry the zero code 8)."""
import numpy as np
import pytest

import oracle
from gen import Workload, activations, config_runs, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gh(lib):
    import gpu_helpers
    return gpu_helpers


def _case(M, K, N, seed=0):
    w = Workload(cfg=9, M=M, K=K, N=N, sparse24=True)
    d = weights(w, seed=3000 + seed + K + N)
    X = activations(w, seed=4000 + seed + M)
    assert oracle.check_24(d["Qp"], K)
    return w, d, X


def _compress(gh, d, K, N):
    import w4a16_mixed_precision_offline_amd as w4
    vp, idx, sp = w4.alloc_sparse24(K, N, 128)
    w4.w4a16_sparse24_repack(gh.dev(d["Qp"]), gh.dev(d["s"]), vp, idx, sp, K, N, 128)
    return vp, idx, sp


def _sgemm(gh, X, comp, M, N, K, variant=-1, splits=0, Y=None):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    vp, idx, sp = comp
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    if variant == -1 and splits == 0:
        w4.w4a16_sparse24_gemm(X, vp, idx, sp, Y, M, N, K, 128)
    else:
        w4.w4a16_sparse24_gemm_plan(X, vp, idx, sp, Y, M, N, K, 128, variant, splits)
    return Y


@pytest.mark.parametrize("K,N", [(256, 32), (1024, 512), (1152, 48)])
def test_compress_matches_layout_model(gh, K, N):
    import layout_model as lm
    _, d, _ = _case(1, K, N)
    vp, idx, sp = _compress(gh, d, K, N)
    mvp, mmeta = lm.sparse24_compress(d["q"], K, N)
    assert np.array_equal(gh.host(vp).view(np.uint32), mvp.reshape(-1))
    assert np.array_equal(gh.host(idx).view(np.uint32), mmeta.reshape(-1))
    assert np.array_equal(gh.host(sp).view(np.uint16), lm.repack_scales(d["s"], N).view(np.uint16))


@pytest.mark.parametrize("K,N", [(4096, 4096), (1152, 48)])
def test_compress_decompress_roundtrip(gh, K, N):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    _, d, _ = _case(1, K, N)
    vp, idx, sp = _compress(gh, d, K, N)
    q = torch.zeros((K // 8, N), dtype=torch.int32, device="cuda")
    s = torch.zeros((K // 128, N), dtype=torch.float16, device="cuda")
    w4.w4a16_sparse24_unpack(vp, idx, sp, q, s, K, N, 128)
    assert np.array_equal(gh.host(q), d["Qp"])
    assert np.array_equal(gh.host(s).view(np.uint16), d["s"].view(np.uint16))


def test_not_24_is_rejected(gh):
    import w4a16_mixed_precision_offline_amd as w4
    _, d, _ = _case(1, 256, 32)
    q = d["q"].copy()
    # make three non-zero codes in one run: positions 0..2 of column 5
    q[0:3, 5] = [1, 2, 3]
    from gen import pack_nibbles_along_k
    d2 = dict(d, Qp=pack_nibbles_along_k(q))
    assert not oracle.check_24(d2["Qp"], 256)
    with pytest.raises(w4.W4A16Error) as e:
        _compress(gh, d2, 256, 32)
    assert e.value.code == -7


def test_onehot_rows_bit_exact(gh):
    K, N = 1024, 256
    _, d, _ = _case(16, K, N)
    ks = [0, 1, 2, 3, 4, 63, 64, 127, 128, 300, 511, 512, 777, 900, 1022, 1023]
    X = np.zeros((16, K), np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], None, K, N, 128)
    Y = gh.host(_sgemm(gh, gh.dev(X), _compress(gh, d, K, N), 16, N, K))
    assert np.array_equal(Y.astype(np.float64), W16[ks].astype(np.float64))


SMALL = [(1, 1024, 512), (5, 1152, 512), (16, 1024, 512), (33, 1280, 512), (64, 1024, 512),
         (100, 1536, 512), (16, 2048, 528), (3, 384, 48)]


@pytest.mark.parametrize("M,K,N", SMALL)
def test_parity_every_variant_and_split(gh, M, K, N):
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N)
    comp = _compress(gh, d, K, N)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], None, 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], None, 128)
    ran = 0
    for v in range(w4.w4a16_gemm_variants()):
        name = w4.w4a16_gemm_variant_name(v)
        # tiled variants take any N % 16; their `splits` is the number of workgroups
        nt = 1 if name.startswith("tiled") else int(name.split("_nt")[1].split("_")[0])
        # the 2:4 tiled kernel needs four column tiles per wave (four-wave 256-column tiles)
        refused = N % (16 * nt) != 0 or (name.startswith("tiled") and ("_bn256_" not in name or
                                                                      "_w8_" in name))
        for splits in (1, 2, 3):
            Y = gh.nan_filled(M, N)
            if refused:
                with pytest.raises(w4.W4A16Error):
                    _sgemm(gh, Xd, comp, M, N, K, variant=v, splits=splits, Y=Y)
                continue
            _sgemm(gh, Xd, comp, M, N, K, variant=v, splits=splits, Y=Y)
            ok, info = oracle.accept(gh.host(Y), Yref, B)
            assert ok, (name, splits, info)
            ran += 1
    assert ran > 0


def test_config4_sparse_and_dense_on_same_weights(gh):
    """Every run of the 2:4 configuration at full size, sparse kernel and dense kernel
    on the same pruned weights; both against the oracle (sampled for large outputs)."""
    cache = {}
    for w in config_runs(4):
        if (w.K, w.N) not in cache:
            cache.clear()
            d = weights(w)
            cache[(w.K, w.N)] = (d, _compress(gh, d, w.K, w.N), gh.repack(d, w.K, w.N))
        d, comp, dense = cache[(w.K, w.N)]
        X = activations(w)
        Xd = gh.dev(X)
        Ys = gh.host(_sgemm(gh, Xd, comp, w.M, w.N, w.K, Y=gh.nan_filled(w.M, w.N)))
        Yd = gh.host(gh.gemm(Xd, dense, w.M, w.N, w.K, Y=gh.nan_filled(w.M, w.N)))
        # every output written (NaN-filled before), then one row per 16-row tile x one
        # column per 16-column tile against the oracle: every output tile is reached
        rows, cols = gh.tile_samples(w.M, w.N)
        Yref, Bd = oracle.gemm_sampled(X, d["Qp"], d["s"], None, 128, rows, cols)
        for Y in (Ys, Yd):
            assert np.all(np.isfinite(Y)), w.name
            ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, Bd)
            assert ok, (w.name, info)


@pytest.mark.parametrize("M,K,N", [(300, 2048, 1040), (130, 1024, 512), (1, 1024, 512)])
def test_tiled_sparse_grids(gh, M, K, N):
    """The tiled kernels in the 2:4 format, at several workgroup counts (stripes cut
    tiles at odd k-blocks); each run repeats bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N)
    comp = _compress(gh, d, K, N)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], None, 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], None, 128)
    # the 2:4 format runs on the tiled variants with four column tiles per wave (256 columns)
    tiled = [v for v in range(w4.w4a16_gemm_variants())
             if w4.w4a16_gemm_variant_name(v).startswith("tiled")
             and "_bn256_" in w4.w4a16_gemm_variant_name(v)
             and "_w8_" not in w4.w4a16_gemm_variant_name(v)]
    assert tiled
    for v in tiled:
        for grid in (0, 1, 3, 6, 16):
            Y = gh.nan_filled(M, N)
            _sgemm(gh, Xd, comp, M, N, K, variant=v, splits=grid, Y=Y)
            first = gh.host(Y).view(np.uint16).copy()
            ok, info = oracle.accept(first.view(np.float16), Yref, B)
            assert ok, (w4.w4a16_gemm_variant_name(v), grid, info)
            Y2 = gh.nan_filled(M, N)
            _sgemm(gh, Xd, comp, M, N, K, variant=v, splits=grid, Y=Y2)
            assert np.array_equal(gh.host(Y2).view(np.uint16), first), (v, grid)


def test_tiled_sparse_onehot_exact(gh):
    """One-hot activation rows through the tiled 2:4 kernel select fp16 weight rows
    exactly: RNE((q - 8) * s) of row k_m."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 200, 1024, 528
    _, d, _ = _case(M, K, N)
    rng = np.random.default_rng(11)
    ks = rng.integers(0, K, size=M)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], None, K, N, 128)
    comp = _compress(gh, d, K, N)
    for v in range(w4.w4a16_gemm_variants()):
        name = w4.w4a16_gemm_variant_name(v)
        if not name.startswith("tiled") or "_bn256_" not in name or "_w8_" in name:
            continue
        for grid in (1, 7):
            Y = gh.host(_sgemm(gh, gh.dev(X), comp, M, N, K, variant=v, splits=grid))
            assert np.array_equal(Y.view(np.uint16), W16[ks].view(np.uint16)), (v, grid)


def test_sparse_refuses_tiles_without_four_column_tiles_per_wave(gh):
    """The 2:4 format's loads are laid out for four column tiles per wave: the 128 x 128
    tiled variant refuses it (an error, nothing launched), and the automatic plan of a
    shape where dense weights take 128 x 128 tiles still runs and matches the oracle."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 128, 5120, 1024
    _, d, X = _case(M, K, N)
    comp = _compress(gh, d, K, N)
    v = [v for v in range(w4.w4a16_gemm_variants())
         if w4.w4a16_gemm_variant_name(v) == "tiled_bm128_bn128_s3"]
    assert v
    with pytest.raises(w4.W4A16Error):
        _sgemm(gh, gh.dev(X), comp, M, N, K, variant=v[0], splits=0)
    Y = gh.host(_sgemm(gh, gh.dev(X), comp, M, N, K))
    Yref = oracle.gemm(X, d["Qp"], d["s"], None, 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], None, 128)
    ok, info = oracle.accept(Y, Yref, B)
    assert ok, info


@pytest.mark.parametrize("group", [256, 1024])
def test_sparse_groups_larger_than_128(gh, group):
    """2:4 weights with a group of 256 rows and with one group spanning K (= 1024):
    compress round-trip bit-exact, and the sparse GEMM (automatic plan, and the skinny and
    tiled variants with a K split / stripes) against the oracle on the pruned codes."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    K, N = 1024, 512
    w = Workload(cfg=9, M=1, K=K, N=N, sparse24=True, group=group)
    d = weights(w, seed=3500 + group)
    assert oracle.check_24(d["Qp"], K, group=group)
    vp, idx, sp = w4.alloc_sparse24(K, N, group)
    w4.w4a16_sparse24_repack(gh.dev(d["Qp"]), gh.dev(d["s"]), vp, idx, sp, K, N, group)
    q = torch.zeros((K // 8, N), dtype=torch.int32, device="cuda")
    s = torch.zeros((K // group, N), dtype=torch.float16, device="cuda")
    w4.w4a16_sparse24_unpack(vp, idx, sp, q, s, K, N, group)
    assert np.array_equal(gh.host(q), d["Qp"])
    assert np.array_equal(gh.host(s).view(np.uint16), d["s"].view(np.uint16))
    for M in (5, 300):
        X = activations(Workload(cfg=9, M=M, K=K, N=N), seed=3600 + M)
        Xd = gh.dev(X)
        Yref = oracle.gemm(X, d["Qp"], d["s"], None, group)
        B = oracle.error_bound(X, d["Qp"], d["s"], None, group)
        for v, sp_ in [(-1, 0), (gh.variant_index("skinny_xr16_nt4_wk4_d2"), 3),
                       (gh.variant_index("tiled_bm128_bn256_s3"), 7)]:
            Y = gh.nan_filled(M, N)
            if v < 0:
                w4.w4a16_sparse24_gemm(Xd, vp, idx, sp, Y, M, N, K, group)
            else:
                w4.w4a16_sparse24_gemm_plan(Xd, vp, idx, sp, Y, M, N, K, group, v, sp_)
            ok, info = oracle.accept(gh.host(Y), Yref, B)
            assert ok, (group, M, v, info)
