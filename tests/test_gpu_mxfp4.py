"""GPU parity of the MXFP4 path (E2M1 weight codes with E8M0 scales per 32 rows along
K, fp8 E4M3 activations; the block scales are applied by the matrix instruction)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from gen import Workload, activations_fp8, weights_mxfp4

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gh(lib):
    import gpu_helpers
    return gpu_helpers


def _case(M, K, N, seed=0):
    w = Workload(cfg=9, M=M, K=K, N=N)
    d = weights_mxfp4(w, seed=5000 + seed + K + N)
    X8, a = activations_fp8(w, seed=6000 + seed + M)
    return d, X8, a


def _pack(gh, d, K, N):
    import w4a16_mixed_precision_offline_amd as w4
    wp, sp = w4.alloc_mx(K, N)
    w4.w4a8_mx_repack(gh.dev(d["Qp"]), gh.dev(d["E"]), wp, sp, K, N)
    return wp, sp


def _mx(gh, X8d, ad, packed, M, N, K, variant=-1, grid=0, Y=None):
    import w4a16_mixed_precision_offline_amd as w4
    wp, sp = packed
    if Y is None:
        Y = gh.nan_filled(M, N)
    if variant == -1 and grid == 0:
        w4.w4a8_mx_gemm(X8d, ad, wp, sp, Y, M, N, K)
    else:
        w4.w4a8_mx_gemm_plan(X8d, ad, wp, sp, Y, M, N, K, variant, grid)
    return Y


def _runs(variant_name, M):
    # fp8 activations need an even number of 16-row tiles; the decode kernel takes M <= 32
    if variant_name.startswith("mx_decode_"):
        return M <= 32
    return not variant_name.startswith("tiled_bm16_")


def _grids(variant_name):
    # the decode kernel has no persistent grid (one workgroup per column tiles)
    return (0,) if variant_name.startswith("mx_decode_") else (0, 1, 3, 16)


@pytest.mark.parametrize("K,N", [(128, 16), (1024, 528), (4096, 4096)])
def test_repack_matches_layout_model(gh, K, N):
    import layout_model as lm
    d, _, _ = _case(1, K, N)
    wp, sp = _pack(gh, d, K, N)
    mw, ms = lm.mx_repack(d["Qp"], d["E"], K, N)
    assert np.array_equal(gh.host(wp).view(np.uint32), mw)
    assert np.array_equal(gh.host(sp), ms)


def test_onehot_rows_bit_exact(gh):
    """x8 = 1.0 at row k (no row scale): Y row m is W[k_m, :] = e2m1(q) * 2^(E - 127), an
    exact fp16 value; rows on both sides of 32-row scale blocks and 128-row k-blocks pin
    the lane layout, the nibble order and the block of each scale.  Every variant that
    takes fp8 activations, at two grids."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 200, 1024, 528
    d, _, _ = _case(M, K, N)
    rng = np.random.default_rng(12)
    ks = np.concatenate([[0, 1, 2, 7, 8, 30, 31, 32, 33, 63, 64, 95, 96, 127, 128, 129, 1023],
                         rng.integers(0, K, size=M - 17)])
    X8 = np.zeros((M, K), np.uint8)
    X8[np.arange(M), ks] = 0x38
    # a sum that starts at +0 turns the -0 of code 8 into +0
    W = oracle.dequant_mxfp4(d["Qp"], d["E"], K, N) + 0.0
    want = W[ks].astype(np.float16)
    assert np.array_equal(want.astype(np.float64), W[ks])  # exact in fp16
    packed = _pack(gh, d, K, N)
    X8d = gh.dev(X8)
    ran = 0
    for v in range(w4.w4a8_mx_variants()):
        name = w4.w4a8_mx_variant_name(v)
        for grid in (1, 7):
            if not _runs(name, M):
                with pytest.raises(w4.W4A16Error):
                    _mx(gh, X8d, None, packed, M, N, K, v, grid)
                continue
            Y = gh.host(_mx(gh, X8d, None, packed, M, N, K, v, grid))
            assert np.array_equal(Y.view(np.uint16), want.view(np.uint16)), (name, grid)
            ran += 1
    assert ran > 0


SMALL = [(1, 128, 16), (5, 1152, 512), (16, 1024, 528), (33, 1280, 512), (64, 1024, 512),
         (100, 1536, 1040), (130, 1024, 512), (300, 2048, 1040), (3, 384, 48), (16, 640, 80),
         (9, 2048, 4112), (24, 640, 80), (32, 1152, 512), (17, 2048, 4112)]


def test_decode_kernel_onehot_rows_bit_exact(gh):
    """The decode kernel (M <= 32): one-hot rows at scale-block and k-block boundaries and
    on the last row give exact fp16 weight rows, for every decode variant, at M = 16 and 32
    (one and two 16-row tiles) and at a ragged M = 7 and 23 (rows past M untouched)."""
    import w4a16_mixed_precision_offline_amd as w4
    K, N = 1280, 80
    d, _, _ = _case(32, K, N, seed=4)
    W = oracle.dequant_mxfp4(d["Qp"], d["E"], K, N) + 0.0
    packed = _pack(gh, d, K, N)
    dec = [v for v in range(w4.w4a8_mx_variants())
           if w4.w4a8_mx_variant_name(v).startswith("mx_decode_")]
    assert dec
    for M, ks in ((16, [0, 31, 32, 63, 64, 127, 128, 255, 256, 640, 641, 1000, 1151, 1152, 1200,
                        1279]), (7, [5, 96, 200, 511, 512, 900, 1278]),
                   (32, list(range(0, 1280, 40))), (23, list(range(3, 1280, 55))[:23])):
        X8 = np.zeros((M, K), np.uint8)
        X8[np.arange(M), ks] = 0x38
        want = W[ks].astype(np.float16)
        for v in dec:
            Y = gh.nan_filled(32, N)
            _mx(gh, gh.dev(X8), None, packed, M, N, K, v, 0, Y=Y)
            Yh = gh.host(Y)
            assert np.array_equal(Yh[:M].view(np.uint16), want.view(np.uint16)), (v, M)
            assert np.isnan(Yh[M:].astype(np.float32)).all(), (v, M)


@pytest.mark.parametrize("M,K,N", SMALL)
def test_parity_every_variant_and_grid(gh, M, K, N):
    import w4a16_mixed_precision_offline_amd as w4
    d, X8, a = _case(M, K, N)
    packed = _pack(gh, d, K, N)
    X8d, ad = gh.dev(X8), gh.dev(a)
    Yref = oracle.gemm_mxfp4(X8, a, d["Qp"], d["E"])
    B = oracle.error_bound_mxfp4(X8, a, d["Qp"], d["E"])
    for v in [-1] + list(range(w4.w4a8_mx_variants())):
        name = "auto" if v < 0 else w4.w4a8_mx_variant_name(v)
        if v >= 0 and not _runs(name, M):
            with pytest.raises(w4.W4A16Error):
                _mx(gh, X8d, ad, packed, M, N, K, v, 0)
            continue
        for grid in ((0,) if v < 0 else _grids(name)):
            Y = _mx(gh, X8d, ad, packed, M, N, K, v, grid)
            first = gh.host(Y).view(np.uint16).copy()
            ok, info = oracle.accept(first.view(np.float16), Yref, B)
            assert ok, (name, grid, info)
            Y2 = _mx(gh, X8d, ad, packed, M, N, K, v, grid)
            assert np.array_equal(gh.host(Y2).view(np.uint16), first), (name, grid)


def test_row_scales_and_no_row_scales(gh):
    M, K, N = 40, 2048, 1024
    d, X8, a = _case(M, K, N, seed=3)
    packed = _pack(gh, d, K, N)
    X8d = gh.dev(X8)
    for sc in (None, a):
        Y = gh.host(_mx(gh, X8d, None if sc is None else gh.dev(sc), packed, M, N, K))
        ok, info = oracle.accept(Y, oracle.gemm_mxfp4(X8, sc, d["Qp"], d["E"]),
                                 oracle.error_bound_mxfp4(X8, sc, d["Qp"], d["E"]))
        assert ok, (sc is None, info)


@pytest.mark.parametrize("M,K,N", [(1, 8192, 10240), (16, 8192, 28672), (32, 8192, 10240),
                                   (24, 28672, 8192), (256, 8192, 10240), (1024, 28672, 8192),
                                   (4096, 8192, 10240), (8, 8192, 28672), (64, 8192, 28672),
                                   (192, 28672, 8192), (192, 8192, 10240)])
def test_full_size_layers_sampled(gh, M, K, N):
    """70B-class layers at decode and prefill sizes, in the launch configuration the
    benchmark times; rows and columns sampled (first, last and random) against the oracle."""
    d, X8, a = _case(M, K, N, seed=9)
    packed = _pack(gh, d, K, N)
    Y = gh.host(_mx(gh, gh.dev(X8), gh.dev(a), packed, M, N, K))
    rng = np.random.default_rng(M + N)
    rows = sorted(set([0, M - 1]) | set(rng.choice(M, size=min(M, 16), replace=False).tolist()))
    cols = sorted(set([0, N - 1]) | set(rng.choice(N, size=64, replace=False).tolist()))
    Yref, Bd = oracle.gemm_mxfp4_sampled(X8, a, d["Qp"], d["E"], rows, cols)
    ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, Bd)
    assert ok, info
    assert np.isfinite(Y.astype(np.float32)).all()


def test_bad_arguments_are_rejected_before_launch(gh):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    K, N, M = 256, 32, 4
    d, X8, a = _case(M, K, N)
    wp, sp = _pack(gh, d, K, N)
    X8d, ad = gh.dev(X8), gh.dev(a)
    Y = gh.nan_filled(M, N)
    cases = [
        lambda: w4.w4a8_mx_gemm(X8d, ad, wp, sp, Y, M, N, 200),         # K % 128
        lambda: w4.w4a8_mx_gemm(X8d, ad, wp, sp, Y, M, 24, K),          # N % 16
        lambda: w4.w4a8_mx_gemm(X8d, ad, wp, sp, Y, 0, N, K),           # M = 0
        lambda: w4.w4a8_mx_gemm(X8d, ad, None, sp, Y, M, N, K),         # NULL codes
        lambda: w4.w4a8_mx_gemm(X8d, ad.data_ptr() + 2, wp, sp, Y, M, N, K),  # unaligned scales
        lambda: w4.w4a8_mx_gemm_plan(X8d, ad, wp, sp, Y, M, N, K, 99, 0),
        lambda: w4.w4a8_mx_gemm_plan(X8d, ad, wp, sp, Y, M, N, K, 0, -1),
        lambda: w4.w4a8_mx_repack(gh.dev(d["Qp"]), gh.dev(d["E"]), wp, sp, 100, N),
        lambda: w4.w4a8_mx_repack(None, gh.dev(d["E"]), wp, sp, K, N),
    ]
    for i, c in enumerate(cases):
        with pytest.raises(w4.W4A16Error):
            c()
    torch.cuda.synchronize()
    assert torch.isnan(Y.float()).all()  # nothing was written


def test_hip_graph_replays_match_eager(gh):
    """Captured MXFP4 launches (decode kernel at one and two row tiles, tiled kernel with
    stream-K stripes and the fixup pass) reproduce the eager result bit for bit on every
    replay, with eager work and synchronizations in between."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    st = torch.cuda.Stream()
    cases = []
    for (M, K, N) in [(1, 4096, 4096), (24, 2048, 4112), (300, 2048, 1040), (130, 1024, 768)]:
        d, X8, a = _case(M, K, N, seed=7)
        cases.append((M, K, N, gh.dev(X8), gh.dev(a), _pack(gh, d, K, N),
                      torch.empty((M, N), dtype=torch.float16, device="cuda")))

    def run_all():
        for (M, K, N, x, s, packed, Y) in cases:
            w4.w4a8_mx_gemm(x, s, packed[0], packed[1], Y, M, N, K)

    with torch.cuda.stream(st):
        run_all()
    torch.cuda.synchronize()
    eager = [gh.host(c[-1]).view(np.uint16).copy() for c in cases]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        run_all()
    torch.cuda.synchronize()
    M3, K3, N3, x3, s3, p3, _ = cases[3]
    for rep in range(4):
        for c in cases:
            c[-1].fill_(0)
        junk = torch.empty((M3, N3), dtype=torch.float16, device="cuda")
        w4.w4a8_mx_gemm(x3, None, p3[0], p3[1], junk, M3, N3, K3)  # eager work between replays
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g.replay()
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert np.array_equal(gh.host(c[-1]).view(np.uint16), e), rep


def test_caller_owned_workspace_sized_by_the_query(gh):
    """A caller-owned workspace of W4A16_WS_COUNTER_BYTES + w4a16_workspace_bytes(M, N, K)
    runs the MXFP4 automatic plan of a shape whose 32-row tiles are all cut into stream-K
    pieces (M = 24 on 28672 x 8192), with the same bits as a library-owned one."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 24, 28672, 8192
    d, X8, a = _case(M, K, N, seed=8)
    packed = _pack(gh, d, K, N)
    X8d, ad = gh.dev(X8), gh.dev(a)
    ref = gh.host(_mx(gh, X8d, ad, packed, M, N, K)).view(np.uint16).copy()
    st = torch.cuda.Stream()
    nbytes = w4.WS_COUNTER_BYTES + w4.w4a16_workspace_bytes(M, N, K)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    w4.w4a16_set_workspace(buf, nbytes, stream=st)
    try:
        for _ in range(2):
            with torch.cuda.stream(st):
                Y = _mx(gh, X8d, ad, packed, M, N, K)
            torch.cuda.synchronize()
            assert np.array_equal(gh.host(Y).view(np.uint16), ref)
    finally:
        w4.w4a16_set_workspace(None, 0, stream=st)
    torch.cuda.synchronize()
