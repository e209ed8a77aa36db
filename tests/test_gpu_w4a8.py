"""GPU parity of the W4A8 entry points (INT4 weights x FP8 E4M3 activations with a
per-row fp32 scale; dingiv.github.io "Marlin", section "CUTLASS W4A8（混合精度）")
against the CPU oracle's fp64 definition on the activations' exact values.

Bit-exact where the result has a single rounding (one-hot rows; unit versus absent
row scales; doubled row scales); otherwise within the oracle's acceptance rule, the
same as for fp16 activations: fp8 x (q - z) products are exact in fp32, so only the
fp32 accumulation and the one fp16 rounding of Y remain.
"""
import numpy as np
import pytest

import oracle
from gen import Workload, activations_fp8, config_runs, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gh(lib):
    import gpu_helpers
    return gpu_helpers


def _case(M, K, N, asym=False, seed=0, cfg=9, group=128):
    w = Workload(cfg=cfg, M=M, K=K, N=N, asym=asym, group=group)
    d = weights(w, seed=7000 + seed + K + N)
    X8, a = activations_fp8(w, seed=8000 + seed + M)
    return d, X8, a


def _gemm8(gh, X8, a, packed, M, N, K, variant=-1, splits=0, rows_alloc=None, group=128):
    """Run w4a8_gemm(_plan); Y is the first M rows of a NaN-filled buffer of
    rows_alloc rows so that writes past row M-1 show up.  Returns (Y[:M], whole)."""
    import w4a16_mixed_precision_offline_amd as w4
    wp, sp, zp = packed
    Yall = gh.nan_filled(rows_alloc or M, N)
    Y = Yall[:M]
    x = gh.dev(X8)
    s = gh.dev(a) if a is not None else None
    if variant == -1 and splits == 0:
        w4.w4a8_gemm(x, s, wp, sp, zp, Y, M, N, K, group)
    else:
        w4.w4a8_gemm_plan(x, s, wp, sp, zp, Y, M, N, K, group, variant, splits)
    whole = gh.host(Yall)
    return whole[:M], whole


def _accept(Y, X8, a, d, rows=None, cols=None, group=128):
    if rows is None:
        Yref = oracle.gemm_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], group)
        B = oracle.error_bound_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], group)
        return oracle.accept(Y, Yref, B)
    Yref, B = oracle.gemm_w4a8_sampled(X8, a, d["Qp"], d["s"], d["Zp"], group, rows, cols)
    return oracle.accept(Y[np.ix_(rows, cols)], Yref, B)


def _sample_idx(rng, n, k):
    idx = set([0, n - 1]) | set(rng.choice(n, size=min(n, k), replace=False).tolist())
    return sorted(idx)


@pytest.mark.parametrize("group", [128, 64])
@pytest.mark.parametrize("asym", [False, True])
def test_w4a8_onehot_exact(gh, asym, group):
    """x8 = 1.0 (code 0x38) at one k per row and a power-of-two row scale select
    RNE_fp16(a * (q - z) * s) bit for bit: the fp8 weights are the exact integers q - z
    and a single term is exact in fp32."""
    M, K, N = 16, 1024, 768
    d, _, _ = _case(M, K, N, asym, group=group)
    ks = [0, 1, 7, 8, 9, 63, 64, 127, 128, 255, 300, 511, 640, 777, 900, 1023]
    X8 = np.zeros((M, K), np.uint8)
    X8[np.arange(M), ks] = 0x38
    a = np.array([2.0 ** ((m % 5) - 2) for m in range(M)], dtype=np.float32)
    W = oracle.dequant(d["Qp"], d["s"], d["Zp"], K, N, group)     # exact (q - z) * s
    exp = (W[ks] * a[:, None].astype(np.float64)).astype(np.float16)  # exact, one rounding
    packed = gh.repack(d, K, N, group)
    for nm, splits in [("skinny_xr16_nt1_wk8_d2", 1), ("skinny_xr16_nt4_wk4_d2", 3),
                       ("skinny_xr16_nt2_wk8_d2", 2), ("skinny_xr16_nt3_wk4_d2", 1)]:
        Y, _ = _gemm8(gh, X8, a, packed, M, N, K, gh.variant_index(nm), splits, group=group)
        assert np.array_equal(Y.view(np.uint16), exp.view(np.uint16)), nm


@pytest.mark.parametrize("M,K,N,asym", [(5, 1152, 528, True), (16, 1024, 512, False),
                                        (33, 2048, 1040, True), (300, 1024, 256, False)])
def test_w4a8_every_variant(gh, M, K, N, asym):
    """Every skinny variant, with and without a K split, including row tails (M = 5,
    33, 300) and column counts that are not a multiple of 64; rows past M untouched."""
    import w4a16_mixed_precision_offline_amd as w4
    d, X8, a = _case(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Yref = oracle.gemm_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], 128)
    ran = 0
    for v in [-1] + list(range(w4.w4a16_gemm_variants())):
        name = w4.w4a16_gemm_variant_name(v) if v >= 0 else "auto"
        if name.startswith("tiled"):
            continue
        nt = 1 if v < 0 else int(name.split("_nt")[1].split("_")[0])
        if N % (16 * nt):
            continue
        for splits in ((0,) if v < 0 else (1, 3)):
            Y, whole = _gemm8(gh, X8, a, packed, M, N, K, v, splits, rows_alloc=M + 2)
            ok, info = oracle.accept(Y, Yref, B)
            assert ok, (name, splits, info)
            assert np.all(np.isnan(whole[M:])), (name, splits)
            ran += 1
    assert ran > 1


def test_w4a8_minimal_shapes(gh):
    for M, K, N, asym in [(1, 128, 16, False), (1, 128, 16, True), (2, 256, 32, False)]:
        d, X8, a = _case(M, K, N, asym)
        Y, _ = _gemm8(gh, X8, a, gh.repack(d, K, N), M, N, K)
        ok, info = _accept(Y, X8, a, d)
        assert ok, (M, K, N, asym, info)


def test_w4a8_row_scale_exact(gh):
    """No row scale equals a unit one bit for bit, and doubling the row scales doubles Y
    bit for bit wherever Y is a normal fp16 number."""
    M, K, N = 16, 4096, 1024
    d, X8, a = _case(M, K, N)
    packed = gh.repack(d, K, N)
    Y0, _ = _gemm8(gh, X8, None, packed, M, N, K)
    Y1, _ = _gemm8(gh, X8, np.ones(M, np.float32), packed, M, N, K)
    assert np.array_equal(Y0.view(np.uint16), Y1.view(np.uint16))
    Ya, _ = _gemm8(gh, X8, a, packed, M, N, K)
    Y2, _ = _gemm8(gh, X8, (a * 2).astype(np.float32), packed, M, N, K)
    normal = (np.abs(Ya.astype(np.float32)) >= 2.0 ** -14) & np.isfinite(Y2)
    assert normal.mean() > 0.99
    assert np.array_equal(Y2[normal].astype(np.float32), 2 * Ya[normal].astype(np.float32))
    ok, info = _accept(Ya, X8, a, d)
    assert ok, info


def test_w4a8_deterministic(gh):
    M, K, N = 8, 11008, 4096
    d, X8, a = _case(M, K, N)
    packed = gh.repack(d, K, N)
    ref, _ = _gemm8(gh, X8, a, packed, M, N, K)
    for _ in range(10):
        Y, _ = _gemm8(gh, X8, a, packed, M, N, K)
        assert np.array_equal(Y.view(np.uint16), ref.view(np.uint16))
    for splits in (2, 5):  # a K split summed across workgroups in slice order
        v = gh.variant_index("skinny_xr8_nt1_wk8_d4")
        Y1, _ = _gemm8(gh, X8, a, packed, M, N, K, v, splits)
        Y2, _ = _gemm8(gh, X8, a, packed, M, N, K, v, splits)
        assert np.array_equal(Y1.view(np.uint16), Y2.view(np.uint16))
        ok, info = _accept(Y1, X8, a, d)
        assert ok, (splits, info)


@pytest.mark.parametrize("cfg", [0, 1, 3])
def test_w4a8_config_shapes(gh, cfg):
    """The tiny, decode-sweep and zero-point configurations' shapes at full size with fp8
    activations (automatic plan, the one bench.py times): small outputs whole, larger
    ones on sampled rows x columns."""
    cache = {}
    for w in config_runs(cfg):
        key = (w.K, w.N)
        if key not in cache:
            d = weights(w)
            cache.clear()
            cache[key] = (d, gh.repack(d, w.K, w.N))
        d, packed = cache[key]
        X8, a = activations_fp8(w)
        Y, _ = _gemm8(gh, X8, a, packed, w.M, w.N, w.K)
        if w.M * w.N <= 16 * 4096:
            ok, info = _accept(Y, X8, a, d)
        else:
            rng = np.random.default_rng(w.M + w.N)
            ok, info = _accept(Y, X8, a, d, _sample_idx(rng, w.M, 24), _sample_idx(rng, w.N, 48))
        assert ok, (w.name, info)


@pytest.mark.parametrize("M,K,N", [(16, 8192, 28672), (256, 8192, 10240), (64, 28672, 8192),
                                   (8, 8192, 28672), (1024, 8192, 10240)])
def test_w4a8_large_layers(gh, M, K, N):
    """70B-class layer shapes (several 64-row blocks at M = 256), sampled outputs."""
    w = Workload(cfg=2, M=M, K=K, N=N, s_lo=0.001, s_hi=0.01)
    d = weights(w)
    X8, a = activations_fp8(w)
    Y, _ = _gemm8(gh, X8, a, gh.repack(d, K, N), M, N, K)
    rng = np.random.default_rng(M + N)
    ok, info = _accept(Y, X8, a, d, _sample_idx(rng, M, 24), _sample_idx(rng, N, 48))
    assert ok, info


@pytest.mark.parametrize("M,K,N,asym", [(5, 1152, 528, True), (33, 2048, 1040, False),
                                        (16, 4096, 11008, True)])
def test_w4a8_groups_of_64(gh, M, K, N, asym):
    """Groups of 64 rows: two scale (and zero-point) rows per 128-row block, one fp32
    partial per half; automatic plan and a spread of explicit variants and K splits."""
    d, X8, a = _case(M, K, N, asym, group=64)
    packed = gh.repack(d, K, N, 64)
    Yref = oracle.gemm_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], 64)
    B = oracle.error_bound_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], 64)
    plans = [(-1, 0), (gh.variant_index("skinny_xr4_nt1_wk8_d4"), 3),
             (gh.variant_index("skinny_xr16_nt2_wk8_d2"), 1),
             (gh.variant_index("skinny_xr32_nt1_wk4_d2"), 2),
             (gh.variant_index("skinny_xr64_nt1_wk4_d2"), 1)]
    for v, splits in plans:
        if v >= 0 and N % (16 * int(gh.w4.w4a16_gemm_variant_name(v).split("_nt")[1].split("_")[0])):
            continue  # this variant's column tiles do not divide N
        Y, whole = _gemm8(gh, X8, a, packed, M, N, K, v, splits, rows_alloc=M + 2, group=64)
        ok, info = oracle.accept(Y, Yref, B)
        assert ok, (v, splits, info)
        assert np.all(np.isnan(whole[M:]))


# ---- tiled kernel (larger M): v_mfma_scale_f32_16x16x128_f8f6f4, fp32 scales per block ----
W4A8_TILED = [(300, 2048, 1040, False), (257, 1536, 512, True), (130, 3072, 272, False),
              (64, 1024, 768, True), (1, 1024, 512, False), (1000, 1024, 2048, True)]


def _tiled_variants(w4):
    # 16-row tiles are odd for fp8 (8 rows per load); the eight-wave 128 x 512 tiles run
    # the fp16-activation formats only (fp8 needs two column tiles per wave there)
    return [v for v in range(w4.w4a16_gemm_variants())
            if w4.w4a16_gemm_variant_name(v).startswith("tiled")
            and not w4.w4a16_gemm_variant_name(v).startswith("tiled_bm16")
            and not w4.w4a16_gemm_variant_name(v).startswith("tiled_bm128_bn512_w8")]


@pytest.mark.parametrize("M,K,N,asym", W4A8_TILED)
def test_w4a8_tiled_grids(gh, M, K, N, asym):
    """Every tiled variant with an even number of 16-row tiles, at workgroup counts that
    leave whole tiles data-parallel and counts that cut tiles into stream-K stripes (the
    row scales then apply in the second pass); each run repeats bit for bit and leaves the
    rows past M untouched."""
    import w4a16_mixed_precision_offline_amd as w4
    d, X8, a = _case(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Yref = oracle.gemm_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], 128)
    tiled = _tiled_variants(w4)
    assert len(tiled) >= 3
    for v in tiled:
        for grid in (0, 1, 3, 5, 8, 24):
            Y, whole = _gemm8(gh, X8, a, packed, M, N, K, v, grid, rows_alloc=M + 2)
            ok, info = oracle.accept(Y, Yref, B)
            assert ok, (w4.w4a16_gemm_variant_name(v), grid, info)
            assert np.all(np.isnan(whole[M:]))
            Y2, _ = _gemm8(gh, X8, a, packed, M, N, K, v, grid)
            assert np.array_equal(Y2.view(np.uint16), Y.view(np.uint16)), (v, grid)


def test_w4a8_tiled_rejects_odd_row_tiles(gh):
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 64, 1024, 512
    d, X8, a = _case(M, K, N)
    packed = gh.repack(d, K, N)
    v16 = [v for v in range(w4.w4a16_gemm_variants())
           if w4.w4a16_gemm_variant_name(v).startswith("tiled_bm16")]
    with pytest.raises(w4.W4A16Error):
        _gemm8(gh, X8, a, packed, M, N, K, v16[0], 0)
    with pytest.raises(w4.W4A16Error):  # eight-wave 128 x 512 tiles: no fp8 mode
        _gemm8(gh, X8, a, packed, M, N, K, gh.variant_index("tiled_bm128_bn512_w8_s2"), 0)
    with pytest.raises(w4.W4A16Error):  # groups of 64: skinny kernel only
        _gemm8(gh, X8, a, gh.repack(_case(M, K, N, group=64)[0], K, N, 64), M, N, K,
               _tiled_variants(w4)[0], 0, group=64)


def test_w4a8_tiled_onehot_exact(gh):
    """One-hot fp8 rows with power-of-two row scales through the tiled kernel (stripes
    included): Y[m, :] = RNE_fp16(a[m] * (q - z) * s) of row k_m bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 200, 1024, 528
    d, _, _ = _case(M, K, N, True)
    rng = np.random.default_rng(8)
    ks = rng.integers(0, K, size=M)
    X8 = np.zeros((M, K), np.uint8)
    X8[np.arange(M), ks] = 0x38
    a = np.array([2.0 ** ((m % 7) - 3) for m in range(M)], dtype=np.float32)
    W = oracle.dequant(d["Qp"], d["s"], d["Zp"], K, N, 128)
    exp = (W[ks] * a[:, None].astype(np.float64)).astype(np.float16)
    packed = gh.repack(d, K, N)
    for v in _tiled_variants(w4):
        for grid in (1, 7):
            Y, _ = _gemm8(gh, X8, a, packed, M, N, K, v, grid)
            assert np.array_equal(Y.view(np.uint16), exp.view(np.uint16)), (v, grid)


def test_w4a8_hip_graph_replays_match_eager(gh):
    """Captured W4A8 launches (skinny with and without a K split, tiled with stream-K
    stripes and the fixup pass) reproduce the eager result bit for bit on every replay,
    with eager work and synchronizations in between."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    st = torch.cuda.Stream()
    plans = [(1, 4096, 4096, -1, 0), (8, 11008, 4096, gh.variant_index("skinny_xr8_nt1_wk8_d4"), 3),
             (300, 2048, 1040, -1, 0), (130, 1024, 768, gh.variant_index("tiled_bm64_bn256_s3"), 7)]
    cases = []
    for (M, K, N, v, sp) in plans:
        d, X8, a = _case(M, K, N, asym=(M % 2 == 0))
        cases.append((M, K, N, v, sp, gh.dev(X8), gh.dev(a), gh.repack(d, K, N),
                      torch.empty((M, N), dtype=torch.float16, device="cuda")))

    def run_all():
        for (M, K, N, v, sp, x, s, packed, Y) in cases:
            w4.w4a8_gemm_plan(x, s, *packed, Y, M, N, K, 128, v, sp)

    with torch.cuda.stream(st):
        run_all()
    torch.cuda.synchronize()
    eager = [gh.host(c[-1]).view(np.uint16).copy() for c in cases]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        run_all()
    torch.cuda.synchronize()
    for rep in range(4):
        for c in cases:
            c[-1].fill_(0)
        junk, _ = _gemm8(gh, np.zeros((2, 1024), np.uint8), None, cases[3][7], 2, 768, 1024)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g.replay()
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert np.array_equal(gh.host(c[-1]).view(np.uint16), e), rep


def test_w4a8_tiled_without_row_scales(gh):
    """The tiled fp8 path with xscale = NULL (scale 1): matches the oracle, and equals a
    run with unit row scales bit for bit, through data-parallel tiles and stream-K pieces."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 257, 1536, 512
    d, X8, _ = _case(M, K, N, asym=True)
    packed = gh.repack(d, K, N)
    ok, info = _accept(_gemm8(gh, X8, None, packed, M, N, K)[0], X8, None, d)
    assert ok, info
    for v in _tiled_variants(w4):
        for grid in (0, 5):
            Y0, _ = _gemm8(gh, X8, None, packed, M, N, K, v, grid)
            Y1, _ = _gemm8(gh, X8, np.ones(M, np.float32), packed, M, N, K, v, grid)
            assert np.array_equal(Y0.view(np.uint16), Y1.view(np.uint16)), (v, grid)
            ok, info = _accept(Y0, X8, None, d)
            assert ok, (v, grid, info)


# ---- above 32 rows: fp8 rows rewritten in fp16 (exact), the fp16 tiled kernel --------------
def _rows16_variants(w4):
    """(index, name) of the fp16 tiled variants on rewritten rows (w4a8_gemm_plan shares
    w4a16_gemm_bf16_plan's numbering)."""
    nb = w4.w4a16_gemm_bf16_variants()
    return [(v, w4.w4a16_gemm_bf16_variant_name(v)) for v in range(nb)
            if w4.w4a16_gemm_bf16_variant_name(v).startswith("rows16_")]


@pytest.mark.parametrize("M,K,N,asym,group", [(300, 2048, 1040, False, 128),
                                              (257, 1536, 512, True, 128),
                                              (130, 1024, 256, True, 64),
                                              (40, 2048, 768, False, 256)])
def test_w4a8_rows16_every_variant_and_grid(gh, M, K, N, asym, group):
    """fp8 rows rewritten in fp16 on the fp16 tiled kernel: every tiled variant (eight-wave
    ones and groups of 64 included) at several workgroup counts, ragged M and N, with row
    scales; nothing is written past row M - 1, and each run repeats bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    d, X8, a = _case(M, K, N, asym, group=group)
    packed = gh.repack(d, K, N, group)
    ran = 0
    for v, name in _rows16_variants(w4):
        for grid in (0, 1, 3, 8, 24):
            Y, whole = _gemm8(gh, X8, a, packed, M, N, K, v, grid, rows_alloc=M + 3, group=group)
            assert np.all(np.isnan(whole[M:].astype(np.float32))), (name, grid)
            ok, info = _accept(Y, X8, a, d, group=group)
            assert ok, (name, grid, info)
            Y2, _ = _gemm8(gh, X8, a, packed, M, N, K, v, grid, group=group)
            assert np.array_equal(Y2.view(np.uint16), Y.view(np.uint16)), (name, grid)
            ran += 1
    assert ran >= 9 * 5
    Y, _ = _gemm8(gh, X8, a, packed, M, N, K, group=group)  # the automatic plan
    ok, info = _accept(Y, X8, a, d, group=group)
    assert ok, ("auto", info)


@pytest.mark.parametrize("asym,group", [(False, 128), (True, 128), (True, 64)])
def test_w4a8_rows16_every_code_exact(gh, asym, group):
    """Every non-NaN E4M3 code, alone in its row, through the fp16 path gives
    RNE_fp16(a * x * RNE_fp16((q - z) * s)) bit for bit (the code's fp16 value is exact, a
    is a power of two or absent): the conversion of all 254 codes is pinned against the
    oracle's decoding.  Outputs below the fp16 normal range are held to one subnormal
    step."""
    import w4a16_mixed_precision_offline_amd as w4
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    M, K, N = len(codes), 1024, 768
    d, _, _ = _case(M, K, N, asym, group=group)
    rng = np.random.default_rng(11)
    ks = rng.integers(0, K, size=M)
    X8 = np.zeros((M, K), np.uint8)
    X8[np.arange(M), ks] = codes
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, group).astype(np.float64)
    vals = oracle.decode_e4m3(codes)
    packed = gh.repack(d, K, N, group)
    rows16 = dict((n, v) for v, n in _rows16_variants(w4))
    for a in (None, np.array([2.0 ** ((m % 7) - 3) for m in range(M)], dtype=np.float32)):
        av = np.ones(M) if a is None else a.astype(np.float64)
        exp = (av[:, None] * vals[:, None] * W16[ks]).astype(np.float16)  # exact, one rounding
        normal = (np.abs(exp) >= np.float16(2.0 ** -14)) | (exp == 0)
        for nm in ["rows16_tiled_bm128_bn256_s3", "rows16_tiled_bm64_bn128_s4",
                   "rows16_tiled_bm128_bn512_w8_s2"]:
            for grid in (0, 5):
                Y, _ = _gemm8(gh, X8, a, packed, M, N, K, rows16[nm], grid, group=group)
                assert np.array_equal(Y[normal], exp[normal]), (nm, grid)
                diff = np.abs(Y[~normal].astype(np.float64) - exp[~normal].astype(np.float64))
                assert np.all(diff <= 2.0 ** -24), (nm, grid)


@pytest.mark.parametrize("M,K,N,asym,group", [(256, 8192, 28672, False, 128),
                                              (1024, 28672, 8192, True, 128),
                                              (48, 8192, 10240, False, 64),
                                              (4096, 28672, 8192, False, 128)])
def test_w4a8_rows16_full_size(gh, M, K, N, asym, group):
    """The automatic plan above 32 rows at 70B-class sizes (fp16 rows; groups of 64 too),
    NaN-filled output, sampled rows x columns against the oracle."""
    d, X8, a = _case(M, K, N, asym, group=group)
    Y, _ = _gemm8(gh, X8, a, gh.repack(d, K, N, group), M, N, K, group=group)
    assert np.all(np.isfinite(Y.astype(np.float32)))
    rows, cols = gh.tile_samples(M, N)
    ok, info = _accept(Y, X8, a, d, rows, cols, group=group)
    assert ok, info
