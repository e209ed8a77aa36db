"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bit-exact where the result is an integer permutation (repack / unpack) or has a
single rounding (one-hot rows, dequantized fp16 weights, power-of-two scales);
otherwise within the acceptance rule of the oracle (relative Frobenius <= 1e-3 and
|Y - Yref| <= 5e-3 * sum_k |X W| + 1e-4).
"""
import numpy as np
import pytest

import oracle
from gen import Workload, activations, config_runs, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gh(lib):
    import gpu_helpers
    return gpu_helpers


def _case(M, K, N, asym=False, seed=0, s_lo=0.002, s_hi=0.02):
    w = Workload(cfg=9, M=M, K=K, N=N, asym=asym, s_lo=s_lo, s_hi=s_hi)
    d = weights(w, seed=1000 + seed + K + N)
    X = activations(w, seed=2000 + seed + M)
    return w, d, X


def _accept(Y, X, d, group=128, rows=None, cols=None):
    if rows is None:
        Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], group)
        B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], group)
        ok, info = oracle.accept(Y, Yref, B)
    else:
        Yref, B = oracle.gemm_sampled(X, d["Qp"], d["s"], d["Zp"], group, rows, cols)
        ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, B)
    return ok, info


# ---- repack ------------------------------------------------------------------------
@pytest.mark.parametrize("K,N,asym", [(1024, 1024, False), (1152, 528, True), (3072, 768, True),
                                      (256, 16, False)])
def test_repack_matches_layout_model(gh, K, N, asym):
    import layout_model as lm
    _, d, _ = _case(1, K, N, asym)
    wp, sp, zp = gh.repack(d, K, N)
    assert np.array_equal(gh.host(wp).view(np.uint32), lm.repack_codes(d["Qp"], K, N))
    assert np.array_equal(gh.host(sp).view(np.uint16), lm.repack_scales(d["s"], N).view(np.uint16))
    if asym:
        assert np.array_equal(gh.host(zp).view(np.uint32), lm.repack_zeros(d["Zp"], N))


@pytest.mark.parametrize("K,N,asym", [(4096, 4096, False), (2560, 2560, True), (1152, 48, True)])
def test_repack_unpack_roundtrip(gh, K, N, asym):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    _, d, _ = _case(1, K, N, asym)
    wp, sp, zp = gh.repack(d, K, N)
    q = torch.zeros((K // 8, N), dtype=torch.int32, device="cuda")
    s = torch.zeros((K // 128, N), dtype=torch.float16, device="cuda")
    z = torch.zeros((K // 128, N // 8), dtype=torch.int32, device="cuda") if asym else None
    w4.w4a16_unpack(wp, sp, zp, q, s, z, K, N, 128)
    assert np.array_equal(gh.host(q), d["Qp"])
    assert np.array_equal(gh.host(s).view(np.uint16), d["s"].view(np.uint16))
    if asym:
        assert np.array_equal(gh.host(z), d["Zp"])


# ---- bit-exact pins ---------------------------------------------------------------
@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("variant", ["skinny_xr16_nt2_wk8_d2", "skinny_xr16_nt3_wk4_d2",
                                     "skinny_xr16_nt4_wk4_d2"])
def test_onehot_rows_bit_exact(gh, asym, splits, variant):
    # a one-hot row of X selects one weight row: Y must equal RNE((q - z) * s) exactly,
    # whether the scale is applied to the fp32 sums (one or two column tiles per wave)
    # or to the fp16 weights (three or more)
    import torch
    K, N = 1024, 768
    _, d, _ = _case(16, K, N, asym)
    ks = [0, 1, 7, 8, 9, 127, 128, 255, 300, 511, 512, 640, 777, 900, 1022, 1023]
    X = np.zeros((16, K), np.float16)
    for m, k in enumerate(ks):
        X[m, k] = 1
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, 128)
    packed = gh.repack(d, K, N)
    Y = gh.gemm(gh.dev(X), packed, 16, N, K, variant=gh.variant_index(variant), splits=splits)
    Yh = gh.host(Y)
    exp = W16[ks]
    assert np.array_equal(Yh.astype(np.float64), exp.astype(np.float64))
    del torch


@pytest.mark.parametrize("asym", [False, True])
def test_scale_doubling_bit_exact(gh, asym):
    K, N, M = 2048, 512, 16
    _, d, X = _case(M, K, N, asym)
    d2 = dict(d)
    d2["s"] = (d["s"].astype(np.float32) * 2).astype(np.float16)
    Xd = gh.dev(X)
    Y1 = gh.host(gh.gemm(Xd, gh.repack(d, K, N), M, N, K)).astype(np.float32)
    Y2 = gh.host(gh.gemm(Xd, gh.repack(d2, K, N), M, N, K)).astype(np.float32)
    normal = np.abs(Y1) >= 2.0 ** -13   # fp16 subnormal outputs do not scale exactly
    assert np.array_equal(Y2[normal], 2 * Y1[normal])


# ---- parity across variants, splits and ragged shapes ----------------------------------
SMALL = [(1, 1024, 512, False), (5, 1152, 512, True), (16, 1024, 512, False),
         (33, 1280, 512, True), (64, 1024, 512, False), (100, 1536, 512, True),
         (16, 2048, 528, False), (3, 384, 48, True)]


@pytest.mark.parametrize("M,K,N,asym", SMALL)
def test_parity_every_variant_and_split(gh, M, K, N, asym):
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], 128)
    ran = 0
    for v in range(w4.w4a16_gemm_variants()):
        name = w4.w4a16_gemm_variant_name(v)
        # tiled variants take any N % 16; their `splits` is the number of workgroups
        nt = 1 if name.startswith("tiled") else int(name.split("_nt")[1].split("_")[0])
        for splits in (1, 2, 3, 7):
            Y = gh.nan_filled(M, N)
            if N % (16 * nt):
                with pytest.raises(w4.W4A16Error):
                    gh.gemm(Xd, packed, M, N, K, variant=v, splits=splits, Y=Y)
                continue
            gh.gemm(Xd, packed, M, N, K, variant=v, splits=splits, Y=Y)
            ok, info = oracle.accept(gh.host(Y), Yref, B)
            assert ok, (name, splits, info)
            ran += 1
    assert ran > 0


# ---- tiled kernel: several row tiles, ragged M and N, stream-K stripes ----------------
TILED = [(300, 2048, 1040, False), (257, 1536, 512, True), (128, 1024, 768, False),
         (1000, 1024, 2048, True), (130, 3072, 272, False), (1, 1024, 512, False),
         (130, 1024, 512, True)]


@pytest.mark.parametrize("M,K,N,asym", TILED)
def test_tiled_parity_grids(gh, M, K, N, asym):
    """Every tiled variant at several workgroup counts: grids that leave whole tiles
    data-parallel, grids that cut tiles into stripes at odd k-blocks (so that one
    workgroup finishes a partial tile and then starts another), and the automatic plan.
    Each grid is run twice and must repeat bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], 128)
    tiled = [v for v in range(w4.w4a16_gemm_variants())
             if w4.w4a16_gemm_variant_name(v).startswith("tiled")]
    assert tiled
    for v in tiled:
        for grid in (0, 1, 3, 5, 6, 8, 16, 24):
            Y = gh.nan_filled(M, N)
            gh.gemm(Xd, packed, M, N, K, variant=v, splits=grid, Y=Y)
            first = gh.host(Y).view(np.uint16).copy()
            ok, info = oracle.accept(first.view(np.float16), Yref, B)
            assert ok, (w4.w4a16_gemm_variant_name(v), grid, info)
            Y2 = gh.nan_filled(M, N)
            gh.gemm(Xd, packed, M, N, K, variant=v, splits=grid, Y=Y2)
            assert np.array_equal(gh.host(Y2).view(np.uint16), first), (v, grid)


def test_tiled_one_hot_is_exact(gh):
    """One-hot activation rows select weight rows: through the tiled kernel (stripes
    included) Y[m, :] must equal RNE((q - z) * s) of row k_m bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 200, 1024, 528
    _, d, _ = _case(M, K, N, True)
    rng = np.random.default_rng(7)
    ks = rng.integers(0, K, size=M)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, 128)
    packed = gh.repack(d, K, N)
    for v in range(w4.w4a16_gemm_variants()):
        if not w4.w4a16_gemm_variant_name(v).startswith("tiled"):
            continue
        for grid in (1, 7):
            Y = gh.host(gh.gemm(gh.dev(X), packed, M, N, K, variant=v, splits=grid))
            assert np.array_equal(Y.view(np.uint16), W16[ks].view(np.uint16)), (v, grid)


def test_config0(gh):
    (w,) = config_runs(0)
    d = weights(w)
    X = activations(w)
    Y = gh.gemm(gh.dev(X), gh.repack(d, w.K, w.N), w.M, w.N, w.K)
    ok, info = _accept(gh.host(Y), X, d)
    assert ok, info


def _sample_idx(rng, n, k):
    idx = set([0, n - 1]) | set(rng.choice(n, size=min(n, k), replace=False).tolist())
    return sorted(idx)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_configs_full_size(gh, cfg):
    """Every run of configs 1-4 at full size, automatic plan (the one bench.py times).
    Y starts NaN-filled and must come back finite everywhere; small outputs are checked
    whole, large ones on one row per 16-row tile x one column per 16-column tile, which
    reaches every output tile and stream-K piece.  Config 4 runs the dense kernel on the
    2:4-pruned weights."""
    runs = config_runs(cfg)
    cache = {}
    for w in runs:
        key = (w.K, w.N)
        if key not in cache:
            cache.clear()
            d = weights(w)
            cache[key] = (d, gh.repack(d, w.K, w.N))
        d, packed = cache[key]
        X = activations(w)
        Yd = gh.nan_filled(w.M, w.N)
        gh.gemm(gh.dev(X), packed, w.M, w.N, w.K, Y=Yd)
        Y = gh.host(Yd)
        assert np.all(np.isfinite(Y)), w.name
        if w.M * w.N * w.K <= 4096 * 4096 * 32:
            ok, info = _accept(Y, X, d)
        else:
            rows, cols = gh.tile_samples(w.M, w.N)
            ok, info = _accept(Y, X, d, rows=rows, cols=cols)
        assert ok, (w.name, info)


# automatic plans at the boundaries of their rules, full 70B-class / configuration-3 sizes:
# 128-row eight-wave tiles at padded row counts (192, 448) and below a full round with two
# pieces per tile (128), 128 x 512 tiles in two rounds of 224 (448), k workgroups per tile on
# a zero-point layer (48, 128 on 13824 x 5120), and the long-K split of the decode kernel (16)
BOUNDARY = [(192, 8192, 28672, False), (448, 8192, 28672, False), (448, 28672, 8192, False),
            (128, 8192, 28672, False), (48, 13824, 5120, True), (128, 13824, 5120, True),
            (16, 28672, 8192, False), (320, 8192, 10240, False)]


@pytest.mark.parametrize("M,K,N,asym", BOUNDARY)
def test_automatic_plans_at_rule_boundaries(gh, M, K, N, asym):
    """NaN-prefilled Y must come back finite everywhere, and match the oracle on one row
    per 16-row tile x one column per 16-column tile (every tile and stream-K piece); a
    second launch repeats the bits."""
    _, d, X = _case(M, K, N, asym, s_lo=0.001, s_hi=0.01)
    packed = gh.repack(d, K, N)
    Xd = gh.dev(X)
    Yd = gh.nan_filled(M, N)
    gh.gemm(Xd, packed, M, N, K, Y=Yd)
    Y = gh.host(Yd)
    assert np.all(np.isfinite(Y)), (M, K, N)
    rows, cols = gh.tile_samples(M, N)
    ok, info = _accept(Y, X, d, rows=rows, cols=cols)
    assert ok, (M, K, N, info)
    Y2 = gh.nan_filled(M, N)
    gh.gemm(Xd, packed, M, N, K, Y=Y2)
    assert np.array_equal(gh.host(Y2).view(np.uint16), Y.view(np.uint16))


def test_determinism_and_guards(gh):
    import torch
    M, K, N = 16, 4096, 4096
    _, d, X = _case(M, K, N)
    packed = gh.repack(d, K, N)
    Xd = gh.dev(X)
    pad = 4096
    buf = torch.full((M * N + 2 * pad,), 31745, dtype=torch.int16, device="cuda")  # 0x7C01
    Y = buf[pad:pad + M * N].view(torch.float16).view(M, N)
    first = None
    for _ in range(20):
        gh.gemm(Xd, packed, M, N, K, Y=Y)
        cur = gh.host(Y).view(np.uint16).copy()
        if first is None:
            first = cur
        assert np.array_equal(cur, first)
    b = gh.host(buf)
    assert np.all(b[:pad] == 31745) and np.all(b[pad + M * N:] == 31745)
    ok, info = _accept(first.view(np.float16), X, d)
    assert ok, info


def test_two_streams_concurrently(gh):
    import torch
    M, K, N = 8, 4096, 4096
    _, d, X = _case(M, K, N)
    packed = gh.repack(d, K, N)
    Xd = gh.dev(X)
    ref = gh.host(gh.gemm(Xd, packed, M, N, K)).view(np.uint16)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for st in (s1, s2, s1, s2):
        with torch.cuda.stream(st):
            outs.append(gh.gemm(Xd, packed, M, N, K))
    torch.cuda.synchronize()
    for Y in outs:
        assert np.array_equal(gh.host(Y).view(np.uint16), ref)


# ---- unfused baseline ---------------------------------------------------------------
@pytest.mark.parametrize("K,N,asym", [(1024, 512, False), (1152, 528, True), (128, 16, True),
                                      (4096, 1040, False)])
def test_dequant_bit_exact(gh, K, N, asym):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    _, d, _ = _case(1, K, N, asym)
    Wt = torch.empty((N, K), dtype=torch.float16, device="cuda")
    w4.w4a16_dequant(gh.dev(d["Qp"]), gh.dev(d["s"]), gh.dev(d["Zp"]) if asym else None, Wt, K, N, 128)
    exp = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, 128).T
    assert np.array_equal(gh.host(Wt).view(np.uint16), np.ascontiguousarray(exp).view(np.uint16))


@pytest.mark.parametrize("M,K,N", [(1, 1024, 512), (16, 4096, 4096), (40, 1152, 528), (128, 1024, 256)])
def test_fp16_gemm_parity(gh, M, K, N):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N)
    Wt = torch.empty((N, K), dtype=torch.float16, device="cuda")
    w4.w4a16_dequant(gh.dev(d["Qp"]), gh.dev(d["s"]), None, Wt, K, N, 128)
    Y = gh.nan_filled(M, N)
    w4.w4a16_fp16_gemm(gh.dev(X), Wt, Y, M, N, K)
    ok, info = _accept(gh.host(Y), X, d)
    assert ok, info


F16_TILED = [(300, 2048, 1040), (257, 1536, 528), (130, 1024, 272), (1, 1024, 512),
             (64, 3072, 128)]


@pytest.mark.parametrize("M,K,N", F16_TILED)
def test_fp16_tiled_parity_grids(gh, M, K, N):
    """The fp16 baseline's tiled variants (fp16 weight tiles, no unpacking) at several
    workgroup counts, ragged M and N included, plus the automatic plan; each grid
    repeats bit for bit."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N)
    Wt = torch.empty((N, K), dtype=torch.float16, device="cuda")
    w4.w4a16_dequant(gh.dev(d["Qp"]), gh.dev(d["s"]), None, Wt, K, N, 128)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], 128)
    tiled = [v for v in range(w4.w4a16_fp16_gemm_variants())
             if w4.w4a16_fp16_gemm_variant_name(v).startswith("tiled_f16")]
    assert len(tiled) >= 2
    runs = [(-1, 0)] + [(v, g) for v in tiled for g in (0, 1, 3, 5, 8, 24)]
    for v, grid in runs:
        Y = gh.nan_filled(M, N)
        w4.w4a16_fp16_gemm_plan(Xd, Wt, Y, M, N, K, v, grid)
        first = gh.host(Y).view(np.uint16).copy()
        ok, info = oracle.accept(first.view(np.float16), Yref, B)
        assert ok, (w4.w4a16_fp16_gemm_variant_name(v) if v >= 0 else "auto", grid, info)
        Y2 = gh.nan_filled(M, N)
        w4.w4a16_fp16_gemm_plan(Xd, Wt, Y2, M, N, K, v, grid)
        assert np.array_equal(gh.host(Y2).view(np.uint16), first), (v, grid)


def test_fp16_tiled_one_hot_is_exact(gh):
    """One-hot rows through the fp16 tiled variants return the fp16 weight rows exactly."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 200, 1024, 528
    _, d, _ = _case(M, K, N)
    rng = np.random.default_rng(8)
    ks = rng.integers(0, K, size=M)
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], None, K, N, 128)
    Wt = torch.from_numpy(np.ascontiguousarray(W16.T)).cuda()
    for v in range(w4.w4a16_fp16_gemm_variants()):
        if not w4.w4a16_fp16_gemm_variant_name(v).startswith("tiled_f16"):
            continue
        for grid in (1, 7):
            Y = gh.nan_filled(M, N)
            w4.w4a16_fp16_gemm_plan(gh.dev(X), Wt, Y, M, N, K, v, grid)
            assert np.array_equal(gh.host(Y).view(np.uint16), W16[ks].view(np.uint16)), (v, grid)


def test_error_codes_on_device(gh):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    X = torch.zeros((4, 1024), dtype=torch.float16, device="cuda")
    Y = torch.zeros((4, 1024), dtype=torch.float16, device="cuda")
    wp, sp, zp = w4.alloc_packed(1024, 1024, 128, False)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm(X, wp, sp, None, Y, 4, 1000, 1024, 128)
    assert e.value.code == -2
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_gemm(X[:, 1:], wp, sp, None, Y, 4, 1024, 1024, 128)
    assert e.value.code == -3


def test_hip_graph_replays_match_eager(gh):
    """The bench times captured HIP graphs: every replay (with eager work and
    synchronizations in between) must reproduce the eager result bit for bit,
    including launches that use the split-K counters."""
    import torch
    shapes = [(1, 4096, 4096), (16, 4096, 11008), (32, 11008, 4096)]
    st = torch.cuda.Stream()
    cases = []
    for (M, K, N) in shapes:
        _, d, X = _case(M, K, N)
        cases.append((M, K, N, gh.dev(X), gh.repack(d, K, N),
                      torch.empty((M, N), dtype=torch.float16, device="cuda")))
    with torch.cuda.stream(st):
        for (M, K, N, Xd, packed, Y) in cases:
            gh.gemm(Xd, packed, M, N, K, Y=Y)
    torch.cuda.synchronize()
    eager = [gh.host(c[5]).view(np.uint16).copy() for c in cases]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for (M, K, N, Xd, packed, Y) in cases:
            gh.gemm(Xd, packed, M, N, K, Y=Y)
    torch.cuda.synchronize()
    for rep in range(5):
        for c in cases:
            c[5].fill_(0)
        junk = gh.gemm(cases[0][3], cases[0][4], 1, 4096, 4096)  # eager work in between
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g.replay()
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert np.array_equal(gh.host(c[5]).view(np.uint16), e), rep
        del junk


def test_graph_keeps_its_workspace_when_the_stream_grows_it(gh):
    """A graph captured with a split-K launch holds the stream's workspace of that time.
    A larger eager launch on the same stream afterwards grows the workspace; the old buffer
    is retired, not freed, so every later replay still reproduces the eager result bit for
    bit.  A capture that would need the workspace to grow is refused before anything is
    enqueued (W4A16_ERR_WORKSPACE)."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    st = torch.cuda.Stream()
    M, K, N = 1, 4096, 256  # skinny kernel, K split across workgroups
    assert w4.w4a16_gemm_describe(M, N, K, 128)["splits"] > 1
    _, d, X = _case(M, K, N)
    Xd, packed = gh.dev(X), gh.repack(d, K, N)
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    with torch.cuda.stream(st):
        gh.gemm(Xd, packed, M, N, K, Y=Y)
    torch.cuda.synchronize()
    eager = gh.host(Y).view(np.uint16).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        gh.gemm(Xd, packed, M, N, K, Y=Y)
    torch.cuda.synchronize()
    # a tiled launch with stream-K pieces (64 MiB of partials) grows the stream's buffer
    Mb, Kb, Nb = 1024, 2048, 4096
    assert w4.w4a16_workspace_bytes(Mb, Nb, Kb) > w4.w4a16_workspace_bytes(M, N, K)
    _, db, Xb = _case(Mb, Kb, Nb)
    Xbd, packedb = gh.dev(Xb), gh.repack(db, Kb, Nb)
    for rep in range(3):
        Yb = torch.empty((Mb, Nb), dtype=torch.float16, device="cuda")
        with torch.cuda.stream(st):
            gh.gemm(Xbd, packedb, Mb, Nb, Kb, Y=Yb)
            Y.fill_(0)
            g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gh.host(Y).view(np.uint16), eager), rep
    rows, cols = gh.tile_samples(Mb, Nb)
    Yref, B = oracle.gemm_sampled(Xb, db["Qp"], db["s"], db["Zp"], 128, rows, cols)
    ok, info = oracle.accept(gh.host(Yb)[np.ix_(rows, cols)], Yref, B)
    assert ok, info
    # a fresh stream has no workspace yet: capturing a split-K launch on it is refused
    st2 = torch.cuda.Stream()
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(w4.W4A16Error) as e:
        with torch.cuda.graph(g2, stream=st2):
            gh.gemm(Xd, packed, M, N, K, Y=Y)
    assert e.value.code == -6


# ---- degenerate and boundary cases ----------------------------------------------------
def _pack_k(q: np.ndarray) -> np.ndarray:
    """uint8 codes [K, N] -> int32 [K/8, N], nibble j of word i = row 8i + j."""
    K, N = q.shape
    w = np.zeros((K // 8, N), np.uint32)
    for j in range(8):
        w |= q[j::8].astype(np.uint32) << np.uint32(4 * j)
    return w.view(np.int32)


def _pack_n(z: np.ndarray) -> np.ndarray:
    """uint8 zero-points [G, N] -> int32 [G, N/8], nibble j of word c = column 8c + j."""
    G, N = z.shape
    w = np.zeros((G, N // 8), np.uint32)
    for j in range(8):
        w |= z[:, j::8].astype(np.uint32) << np.uint32(4 * j)
    return w.view(np.int32)


@pytest.mark.parametrize("asym", [False, True])
def test_codes_equal_to_zero_points_give_exact_zero(gh, asym):
    """q = z everywhere makes W = 0: Y must be exactly zero on every kernel path (skinny
    with and without a K split, tiled with stream-K pieces), for any activations."""
    import w4a16_mixed_precision_offline_amd as w4
    K, N = 2048, 528
    rng = np.random.default_rng(11)
    G = K // 128
    z = rng.integers(0, 16, size=(G, N), dtype=np.uint8) if asym else np.full((G, N), 8, np.uint8)
    q = np.repeat(z, 128, axis=0)
    s = rng.uniform(0.002, 0.02, size=(G, N)).astype(np.float32).astype(np.float16)
    d = dict(Qp=_pack_k(q), s=s, Zp=_pack_n(z) if asym else None)
    packed = gh.repack(d, K, N)
    tiled = [v for v in range(w4.w4a16_gemm_variants())
             if w4.w4a16_gemm_variant_name(v).startswith("tiled")]
    for M in (1, 16, 300):
        X = rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)
        Xd = gh.dev(X)
        runs = [(-1, 0), (gh.variant_index("skinny_xr16_nt1_wk4_d4"), 3)] + [(v, 7) for v in tiled]
        for v, sp in runs:
            Y = gh.nan_filled(M, N)
            gh.gemm(Xd, packed, M, N, K, variant=v, splits=sp, Y=Y)
            assert np.all(gh.host(Y).astype(np.float32) == 0.0), (M, v, sp)


@pytest.mark.parametrize("M,K,N,asym", [(1, 128, 16, False), (300, 128, 16, True), (17, 256, 32, False)])
def test_minimal_shapes_every_variant(gh, M, K, N, asym):
    """One 128-row group and one or two 16-column tiles, through every variant that
    accepts the shape (a tile of 16 columns, a single k-block, ragged rows)."""
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], 128)
    ran = 0
    for v in range(w4.w4a16_gemm_variants()):
        name = w4.w4a16_gemm_variant_name(v)
        nt = 1 if name.startswith("tiled") else int(name.split("_nt")[1].split("_")[0])
        if N % (16 * nt):
            continue
        for splits in (0, 1, 2):
            Y = gh.nan_filled(M, N)
            gh.gemm(Xd, packed, M, N, K, variant=v, splits=splits, Y=Y)
            ok, info = oracle.accept(gh.host(Y), Yref, B)
            assert ok, (name, splits, info)
            ran += 1
    assert ran > 0


def test_offsets_past_2_gib_use_the_skinny_kernel(gh):
    """K = 2^23 at M = 256: a 128-row tile of X spans 2 GiB, past the tiled kernel's 32-bit
    buffer offsets, so the automatic plan runs the skinny kernel (64-row blocks, K split
    across workgroups); sampled outputs against the oracle."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 256, 1 << 23, 16
    plan = w4.w4a16_gemm_describe(M, N, K, 128)
    assert plan["name"].startswith("skinny"), plan
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    X = torch.randn((M, K), device="cuda", generator=g).half()
    q = torch.randint(-2 ** 31, 2 ** 31 - 1, (K // 8, N), dtype=torch.int32, device="cuda", generator=g)
    s = (torch.rand((K // 128, N), device="cuda", generator=g) * 0.018 + 0.002).half()
    wp, sp, _ = w4.alloc_packed(K, N, 128, False)
    w4.w4a16_repack(q, s, None, wp, sp, None, K, N, 128)
    Y = gh.nan_filled(M, N)
    w4.w4a16_gemm(X, wp, sp, None, Y, M, N, K, 128)
    rows = [0, 63, 64, 255]
    Xr = gh.host(X[rows])
    del X
    Qp, sh = gh.host(q), gh.host(s)
    Yref, B = oracle.gemm_sampled(Xr, Qp, sh, None, 128, list(range(4)),
                                  list(range(N)))
    ok, info = oracle.accept(gh.host(Y)[rows], Yref, B)
    assert ok, info


# ---- groups of 64 rows (two scale / zero-point rows per 128-row block) -------------------
def _case64(M, K, N, asym=False, seed=0):
    w = Workload(cfg=9, M=M, K=K, N=N, group=64, asym=asym)
    d = weights(w, seed=3000 + seed + K + N)
    X = activations(w, seed=4000 + seed + M)
    return w, d, X


@pytest.mark.parametrize("asym", [False, True])
def test_group64_repack_layout_and_roundtrip(gh, asym):
    import torch
    import layout_model as lm
    import w4a16_mixed_precision_offline_amd as w4
    K, N = 1152, 528
    _, d, _ = _case64(1, K, N, asym)
    wp, sp, zp = gh.repack(d, K, N, 64)
    assert np.array_equal(gh.host(wp).view(np.uint32), lm.repack_codes(d["Qp"], K, N))
    assert np.array_equal(gh.host(sp).view(np.uint16), lm.repack_scales64(d["s"], N).view(np.uint16))
    if asym:
        assert np.array_equal(gh.host(zp).view(np.uint32), lm.repack_zeros64(d["Zp"], N))
    q = torch.zeros((K // 8, N), dtype=torch.int32, device="cuda")
    s = torch.zeros((K // 64, N), dtype=torch.float16, device="cuda")
    z = torch.zeros((K // 64, N // 8), dtype=torch.int32, device="cuda") if asym else None
    w4.w4a16_unpack(wp, sp, zp, q, s, z, K, N, 64)
    assert np.array_equal(gh.host(q), d["Qp"])
    assert np.array_equal(gh.host(s).view(np.uint16), d["s"].view(np.uint16))
    if asym:
        assert np.array_equal(gh.host(z), d["Zp"])


@pytest.mark.parametrize("M,K,N,asym", [(5, 1152, 528, True), (33, 1024, 512, False),
                                        (300, 2048, 1040, True), (1, 256, 48, False)])
def test_group64_every_variant(gh, M, K, N, asym):
    import w4a16_mixed_precision_offline_amd as w4
    _, d, X = _case64(M, K, N, asym)
    packed = gh.repack(d, K, N, 64)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], 64)
    B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], 64)
    ran = 0
    for v in [-1] + list(range(w4.w4a16_gemm_variants())):
        name = w4.w4a16_gemm_variant_name(v) if v >= 0 else "auto"
        nt = 1 if not name.startswith("skinny") else int(name.split("_nt")[1].split("_")[0])
        if N % (16 * nt):
            continue
        for splits in ((0,) if v < 0 else (1, 3)):
            Y = gh.nan_filled(M, N)
            gh.gemm(Xd, packed, M, N, K, group=64, variant=v, splits=splits, Y=Y)
            ok, info = oracle.accept(gh.host(Y), Yref, B)
            assert ok, (name, splits, info)
            ran += 1
    assert ran > 1


@pytest.mark.parametrize("asym", [False, True])
def test_group64_onehot_exact(gh, asym):
    """One-hot rows in both 64-row halves of a block select RNE((q - z) * s) of their own
    group, through the fp32-rescale and the fp16-scaled-weight skinny paths and the tiled
    kernel."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 16, 1024, 768
    _, d, _ = _case64(M, K, N, asym)
    ks = [0, 1, 63, 64, 65, 127, 128, 191, 192, 300, 511, 512, 575, 640, 1000, 1023]
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, 64)
    packed = gh.repack(d, K, N, 64)
    names = ["skinny_xr16_nt2_wk8_d2", "skinny_xr16_nt3_wk4_d2", "skinny_xr16_nt4_wk4_d2",
             "tiled_bm128_bn256_s3", "tiled_bm64_bn256_s3", "tiled_bm16_bn256_s4"]
    for nm in names:
        for splits in (1, 3):
            Y = gh.host(gh.gemm(gh.dev(X), packed, M, N, K, group=64,
                                variant=gh.variant_index(nm), splits=splits))
            assert np.array_equal(Y.view(np.uint16), W16[ks].view(np.uint16)), (nm, splits)


@pytest.mark.parametrize("M,K,N,asym", [(1, 4096, 11008, False), (16, 4096, 11008, True),
                                        (32, 11008, 4096, False), (1024, 8192, 10240, True)])
def test_group64_full_size(gh, M, K, N, asym):
    _, d, X = _case64(M, K, N, asym)
    Y = gh.host(gh.gemm(gh.dev(X), gh.repack(d, K, N, 64), M, N, K, group=64,
                        Y=gh.nan_filled(M, N)))
    assert np.all(np.isfinite(Y))
    rows, cols = gh.tile_samples(M, N)
    Yref, B = oracle.gemm_sampled(X, d["Qp"], d["s"], d["Zp"], 64, rows, cols)
    ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, B)
    assert ok, info


# ---- bf16 activations (skinny kernel up to 32 rows, tiled above; Y rounded once to bf16) -
BF16_FRO = 4e-3  # one bf16 rounding of Y costs up to 2^-9 of |Y|: the Frobenius limit is 4x looser


def _bf16_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _f32_bf16_rne(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _case_bf16(M, K, N, asym=False, seed=0, group=128):
    from gen import activations_bf16
    w = Workload(cfg=9, M=M, K=K, N=N, asym=asym, group=group)
    d = weights(w, seed=5000 + seed + K + N)
    bits, vals = activations_bf16(w, seed=6000 + seed + M)
    return w, d, bits, vals


def _gemm_bf16(gh, Xbits, packed, M, N, K, variant=-1, splits=0, group=128):
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    wp, sp, zp = packed
    Y = torch.full((M, N), -1, dtype=torch.int16, device="cuda")  # 0xFFFF: a bf16 NaN
    w4.w4a16_gemm_bf16_plan(gh.dev(Xbits.view(np.int16)), wp, sp, zp, Y, M, N, K, group, variant,
                            splits)
    return gh.host(Y).view(np.uint16)


@pytest.mark.parametrize("M,K,N,asym", [(5, 1152, 528, True), (16, 1024, 512, False),
                                        (33, 2048, 1040, True), (300, 1024, 256, False)])
def test_bf16_every_variant(gh, M, K, N, asym):
    import w4a16_mixed_precision_offline_amd as w4
    _, d, bits, vals = _case_bf16(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Yref = oracle.gemm(vals, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound(vals, d["Qp"], d["s"], d["Zp"], 128)
    ran = 0
    for v in [-1] + list(range(w4.w4a16_gemm_variants())):
        name = w4.w4a16_gemm_variant_name(v) if v >= 0 else "auto"
        if name.startswith("tiled"):
            continue
        nt = 1 if v < 0 else int(name.split("_nt")[1].split("_")[0])
        if N % (16 * nt):
            continue
        for splits in ((0,) if v < 0 else (1, 3)):
            Y = _bf16_f32(_gemm_bf16(gh, bits, packed, M, N, K, v, splits))
            ok, info = oracle.accept(Y, Yref, B, rel_fro=BF16_FRO)
            assert ok, (name, splits, info)
            ran += 1
    assert ran > 1


@pytest.mark.parametrize("asym", [False, True])
def test_bf16_onehot_exact(gh, asym):
    """One-hot bf16 rows select RNE_bf16((q - z) * s) bit for bit: the offset removal
    with the activation row sums and the fp32 scale are exact for a single term."""
    M, K, N = 16, 1024, 768
    _, d, _, _ = _case_bf16(M, K, N, asym)
    ks = [0, 1, 7, 8, 9, 127, 128, 255, 300, 511, 512, 640, 777, 900, 1022, 1023]
    bits = np.zeros((M, K), np.uint16)
    bits[np.arange(M), ks] = 0x3F80  # 1.0
    W = oracle.dequant(d["Qp"], d["s"], d["Zp"], K, N, 128)  # exact (q - z) * s
    exp = _f32_bf16_rne(W[ks].astype(np.float32))              # exact in fp32, one rounding
    packed = gh.repack(d, K, N)
    for nm, splits in [("skinny_xr16_nt1_wk8_d2", 1), ("skinny_xr16_nt4_wk4_d2", 3),
                       ("skinny_xr16_nt2_wk8_d2", 2)]:
        Y = _gemm_bf16(gh, bits, packed, M, N, K, gh.variant_index(nm), splits)
        assert np.array_equal(Y, exp), nm


@pytest.mark.parametrize("M,K,N,asym", [(300, 2048, 1040, False), (257, 1536, 512, True),
                                        (130, 1024, 256, True), (64, 1024, 512, False)])
def test_bf16_tiled_every_variant_and_grid(gh, M, K, N, asym):
    """bf16 activations on the tiled kernel: every four-wave tiled variant at several
    workgroup counts (whole tiles, stream-K stripes at odd k-blocks), ragged M and N; the
    eight-wave variants are refused before any launch.  Each run repeats bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    _, d, bits, vals = _case_bf16(M, K, N, asym)
    packed = gh.repack(d, K, N)
    Yref = oracle.gemm(vals, d["Qp"], d["s"], d["Zp"], 128)
    B = oracle.error_bound(vals, d["Qp"], d["s"], d["Zp"], 128)
    ran = 0
    for v in range(w4.w4a16_gemm_variants()):
        name = w4.w4a16_gemm_variant_name(v)
        if not name.startswith("tiled"):
            continue
        if "_w8_" in name:
            with pytest.raises(w4.W4A16Error):
                _gemm_bf16(gh, bits, packed, M, N, K, v, 0)
            continue
        for grid in (0, 1, 3, 5, 8, 24):
            Y1 = _gemm_bf16(gh, bits, packed, M, N, K, v, grid)
            ok, info = oracle.accept(_bf16_f32(Y1), Yref, B, rel_fro=BF16_FRO)
            assert ok, (name, grid, info)
            assert np.array_equal(_gemm_bf16(gh, bits, packed, M, N, K, v, grid), Y1), (name, grid)
            ran += 1
    assert ran >= 6 * 7


@pytest.mark.parametrize("asym", [False, True])
def test_bf16_tiled_onehot_exact(gh, asym):
    """One-hot bf16 rows through the tiled kernel select RNE_bf16((q - z) * s) bit for bit,
    with whole tiles and with stream-K pieces (the second pass writes bf16 too)."""
    M, K, N = 16, 1024, 768
    _, d, _, _ = _case_bf16(M, K, N, asym)
    ks = [0, 1, 7, 8, 9, 127, 128, 255, 300, 511, 512, 640, 777, 900, 1022, 1023]
    bits = np.zeros((M, K), np.uint16)
    bits[np.arange(M), ks] = 0x3F80  # 1.0
    W = oracle.dequant(d["Qp"], d["s"], d["Zp"], K, N, 128)
    exp = _f32_bf16_rne(W[ks].astype(np.float32))
    packed = gh.repack(d, K, N)
    for nm in ["tiled_bm16_bn256_s4", "tiled_bm64_bn128_s4", "tiled_bm128_bn256_s3",
               "tiled_bm128_bn128_s3"]:
        for grid in (1, 7):
            Y = _gemm_bf16(gh, bits, packed, M, N, K, gh.variant_index(nm), grid)
            assert np.array_equal(Y, exp), (nm, grid)


def _rows16_variants(w4):
    """(index, name) of the fp16 tiled variants on rows rewritten in fp16."""
    nb = w4.w4a16_gemm_bf16_variants()
    return [(v, w4.w4a16_gemm_bf16_variant_name(v)) for v in range(nb)
            if w4.w4a16_gemm_bf16_variant_name(v).startswith("rows16_")]


@pytest.mark.parametrize("M,K,N,asym,group", [(300, 2048, 1040, False, 128),
                                              (257, 1536, 512, True, 128),
                                              (130, 1024, 256, True, 64),
                                              (64, 1024, 512, False, 256),
                                              (40, 2048, 768, True, 64)])
def test_bf16_rows16_every_variant_and_grid(gh, M, K, N, asym, group):
    """bf16 rows rewritten in fp16 (a power of two per row) on the fp16 tiled kernel: every
    tiled variant, eight-wave ones and groups of 64 included, at several workgroup counts
    (whole tiles, stream-K stripes), ragged M and N.  Each run repeats bit for bit."""
    import w4a16_mixed_precision_offline_amd as w4
    _, d, bits, vals = _case_bf16(M, K, N, asym, group=group)
    packed = gh.repack(d, K, N, group)
    Yref = oracle.gemm(vals, d["Qp"], d["s"], d["Zp"], group)
    B = oracle.error_bound(vals, d["Qp"], d["s"], d["Zp"], group)
    ran = 0
    for v, name in _rows16_variants(w4):
        for grid in (0, 1, 3, 8, 24):
            Y1 = _gemm_bf16(gh, bits, packed, M, N, K, v, grid, group=group)
            ok, info = oracle.accept(_bf16_f32(Y1), Yref, B, rel_fro=BF16_FRO)
            assert ok, (name, grid, info)
            assert np.array_equal(_gemm_bf16(gh, bits, packed, M, N, K, v, grid, group=group),
                                  Y1), (name, grid)
            ran += 1
    assert ran >= 9 * 5
    # the automatic plan (rows16 where w4a16_gemm takes the tiled kernel)
    Y = _bf16_f32(_gemm_bf16(gh, bits, packed, M, N, K, -1, 0, group=group))
    ok, info = oracle.accept(Y, Yref, B, rel_fro=BF16_FRO)
    assert ok, ("auto", info)


@pytest.mark.parametrize("asym,group", [(False, 128), (True, 128), (True, 64)])
def test_bf16_rows16_onehot_exact(gh, asym, group):
    """One-hot bf16 rows through the fp16 path select RNE_bf16(RNE_fp16((q - z) * s)) bit
    for bit: the row scale 2^15 and its inverse are exact, the weight is the fp16 one of
    w4a16_gemm, and Y is rounded once from it to bf16."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 16, 1024, 768
    _, d, _, _ = _case_bf16(M, K, N, asym, group=group)
    ks = [0, 1, 7, 8, 9, 63, 64, 128, 255, 300, 511, 512, 640, 777, 900, 1023]
    bits = np.zeros((M, K), np.uint16)
    bits[np.arange(M), ks] = 0x3F80  # 1.0
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, group)
    exp = _f32_bf16_rne(W16[ks].astype(np.float32))
    packed = gh.repack(d, K, N, group)
    rows16 = dict((n, v) for v, n in _rows16_variants(w4))
    for nm in ["rows16_tiled_bm16_bn256_s4", "rows16_tiled_bm64_bn128_s4",
               "rows16_tiled_bm128_bn256_s3", "rows16_tiled_bm128_bn512_w8_s2"]:
        for grid in (1, 7):
            Y = _gemm_bf16(gh, bits, packed, M, N, K, rows16[nm], grid, group=group)
            assert np.array_equal(Y, exp), (nm, grid)


def test_bf16_power_of_two_rows_zero_rows_and_outliers(gh):
    """Every bf16 path: a row times 2^k gives exactly 2^k times that row's output, for k
    from -60 to 60, and an all-zero row gives zeros.  A row holding one value far above the
    rest passes the oracle's test within each path's range: 2^24 above the rest on fp16
    rows (exact within 2^32 of the row's maximum), 2^12 on the bf16 variants (the offset
    128 + z leaves the block's fp32 sums, which carry the large value times 128 + q; the
    error reaches the elementwise limit near 2^18)."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 96, 4096, 8192  # 32 Mi weights: the automatic plan takes fp16 rows
    _, d, bits, vals = _case_bf16(M, K, N, True)
    packed = gh.repack(d, K, N)
    base = bits[0].copy()
    ks = [-60, -33, -20, -1, 0, 1, 20, 33, 60]
    rows = np.tile(base, (M, 1))
    for i in range(M):
        k = ks[i % len(ks)]
        e = ((rows[i] >> 7) & 0xFF).astype(np.int32)
        nz = e > 0
        rows[i][nz] = (rows[i][nz] & 0x807F) | ((e[nz] + k).astype(np.uint16) << 7)
    rows[5] = 0
    rows[6, :] = bits[1]
    rows[6, 17] = (rows[6, 17] & 0x8000) | ((127 + 24) << 7) | 0x40  # +-1.5 * 2^24
    rows[7, :] = bits[2]
    rows[7, 40] = (rows[7, 40] & 0x8000) | ((127 + 12) << 7) | 0x40  # +-1.5 * 2^12

    def check_row(Y, i, v):
        vi = _bf16_f32(rows[i:i + 1]).astype(np.float64)
        Yref = oracle.gemm(vi, d["Qp"], d["s"], d["Zp"], 128)
        B = oracle.error_bound(vi, d["Qp"], d["s"], d["Zp"], 128)
        ok, info = oracle.accept(_bf16_f32(Y[i:i + 1]), Yref, B, rel_fro=BF16_FRO)
        assert ok, (v, i, info)

    rows16 = [v for v, n in _rows16_variants(w4) if n in ("rows16_tiled_bm128_bn256_s3",
                                                          "rows16_tiled_bm64_bn128_s4")]
    native = [gh.variant_index("skinny_xr16_nt2_wk8_d2"), gh.variant_index("tiled_bm128_bn256_s3")]
    for v in [-1] + rows16 + native:
        Y = _gemm_bf16(gh, rows, packed, M, N, K, v, 0 if v < 0 else 5)
        y0 = _bf16_f32(Y[ks.index(0)])
        for i in range(M):
            if i in (5, 6, 7):
                continue
            k = ks[i % len(ks)]
            assert np.array_equal(_bf16_f32(Y[i]), y0 * np.float32(2.0 ** k)), (v, i, k)
        assert np.all(_bf16_f32(Y[5]) == 0), v
        check_row(Y, 7, v)
        if v not in native:
            check_row(Y, 6, v)


def test_bf16_rows16_caller_owned_workspace(gh):
    """The fp16 rows of w4a16_gemm_bf16 live in the stream's workspace: a caller-owned buffer
    of W4A16_WS_COUNTER_BYTES + w4a16_workspace_bytes(M, N, K) runs the automatic plan with
    the same bits as a library-owned one, twice in a row; the smallest accepted buffer is
    refused with W4A16_ERR_WORKSPACE before any launch."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 300, 2048, 1040
    _, d, bits, vals = _case_bf16(M, K, N, True)
    packed = gh.repack(d, K, N)
    ref = _gemm_bf16(gh, bits, packed, M, N, K)
    need = w4.w4a16_workspace_bytes(M, N, K)
    assert need >= M * K * 2 + M * 4
    st = torch.cuda.Stream()
    nbytes = w4.WS_COUNTER_BYTES + need
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    w4.w4a16_set_workspace(buf, nbytes, stream=st)
    try:
        for _ in range(2):
            with torch.cuda.stream(st):
                Y = _gemm_bf16(gh, bits, packed, M, N, K)
            torch.cuda.synchronize()
            assert np.array_equal(Y, ref)
    finally:
        w4.w4a16_set_workspace(None, 0, stream=st)
    small = torch.empty(w4.WS_COUNTER_BYTES + 256, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    w4.w4a16_set_workspace(small, small.numel(), stream=st)
    try:
        with torch.cuda.stream(st):
            with pytest.raises(w4.W4A16Error) as e:
                _gemm_bf16(gh, bits, packed, M, N, K)
        assert e.value.code == -6
    finally:
        w4.w4a16_set_workspace(None, 0, stream=st)
    torch.cuda.synchronize()


def test_bf16_rows16_hip_graph_replays_match_eager(gh):
    """Captured bf16 launches above 32 rows (row conversion, fp16 tiled kernel with stream-K
    pieces and the fixup pass, groups of 128 and 64) and one skinny launch reproduce the
    eager result bit for bit on every replay, with eager work and synchronizations between
    the replays."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    st = torch.cuda.Stream()
    plans = [(300, 2048, 1040, 128, -1, 0), (64, 4096, 8192, 64, -1, 0), (16, 1024, 768, 128, -1, 0),
             (130, 1024, 768, 128,
              [v for v in range(w4.w4a16_gemm_bf16_variants())
               if w4.w4a16_gemm_bf16_variant_name(v) == "rows16_tiled_bm64_bn256_s3"][0], 7)]
    cases = []
    for (M, K, N, group, v, sp) in plans:
        _, d, bits, _ = _case_bf16(M, K, N, asym=(M % 2 == 0), group=group)
        cases.append((M, K, N, group, v, sp, gh.dev(bits.view(np.int16)), gh.repack(d, K, N, group),
                      torch.empty((M, N), dtype=torch.int16, device="cuda")))

    def run_all():
        for (M, K, N, group, v, sp, x, packed, Y) in cases:
            w4.w4a16_gemm_bf16_plan(x, *packed, Y, M, N, K, group, v, sp)

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
        _gemm_bf16(gh, np.zeros((40, 1024), np.uint16), cases[3][7], 40, 768, 1024)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            g.replay()
        torch.cuda.synchronize()
        for c, e in zip(cases, eager):
            assert np.array_equal(gh.host(c[-1]).view(np.uint16), e), rep


@pytest.mark.parametrize("asym", [False, True])
def test_bf16_rows16_rows_longer_than_registers(gh, asym):
    """Rows of more than 32768 values do not fit the conversion's registers and are read
    twice (maximum, then conversion): K = 33024 and 65536 on explicit fp16-row variants,
    whole output against the oracle, one row holding a value 2^20 above the rest."""
    import w4a16_mixed_precision_offline_amd as w4
    rows16 = dict((n, v) for v, n in _rows16_variants(w4))
    for (M, K, N) in [(40, 33024, 256), (17, 65536, 128)]:
        _, d, bits, vals = _case_bf16(M, K, N, asym)
        bits = bits.copy()
        bits[3, K - 5] = (bits[3, K - 5] & 0x8000) | ((127 + 20) << 7)  # +-2^20, near the end
        vals = _bf16_f32(bits).astype(np.float64)
        packed = gh.repack(d, K, N)
        Yref = oracle.gemm(vals, d["Qp"], d["s"], d["Zp"], 128)
        B = oracle.error_bound(vals, d["Qp"], d["s"], d["Zp"], 128)
        for nm, grid in [("rows16_tiled_bm64_bn128_s4", 0), ("rows16_tiled_bm16_bn256_s4", 7)]:
            Y = _bf16_f32(_gemm_bf16(gh, bits, packed, M, N, K, rows16[nm], grid))
            ok, info = oracle.accept(Y, Yref, B, rel_fro=BF16_FRO)
            assert ok, (M, K, nm, info)


def _bf16_bits(sign, exp_unbiased, mant7):
    return np.uint16((sign << 15) | ((exp_unbiased + 127) << 7) | mant7)


def test_bf16_rows16_exact_range_of_a_row(gh):
    """The fp16 rows carry every value within 2^32 of the row's maximum exactly.  Each row
    holds its maximum 1.5 * 2^E and one value (255/128) * 2^(E - delta) with all eight
    significant bits set; in the columns whose weight at the maximum's position is zero the
    output is that value times the fp16 weight alone, so it must equal
    RNE_bf16(value * RNE_fp16((q - z) * s)) bit for bit for delta = 1 .. 32 (the smallest
    carried exactly lands on the fp16 subnormal grid), over maxima from 2^-60 to 2^100."""
    import w4a16_mixed_precision_offline_amd as w4
    M, K, N = 64, 1024, 768
    _, d, _, _ = _case_bf16(M, K, N, False)
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, 128).astype(np.float64)
    rng = np.random.default_rng(12)
    Es = [-60, -40, -3, 0, 7, 25, 60, 100]
    deltas = [1, 2, 7, 8, 15, 16, 23, 24, 30, 31, 32]
    bits = np.zeros((M, K), np.uint16)
    big_k, small_k, small_v = [], [], []
    for r in range(M):
        E = Es[r % len(Es)]
        delta = deltas[r % len(deltas)]
        k1, k2 = rng.choice(K, size=2, replace=False)
        bits[r, k1] = _bf16_bits(r % 2, E, 0x40)                   # 1.5 * 2^E
        bits[r, k2] = _bf16_bits((r // 2) % 2, E - delta, 0x7F)    # (255/128) * 2^(E - delta)
        big_k.append(k1)
        small_k.append(k2)
        small_v.append(float(_bf16_f32(bits[r, k2:k2 + 1])[0]))
    packed = gh.repack(d, K, N)
    rows16 = dict((n, v) for v, n in _rows16_variants(w4))
    for nm in ["rows16_tiled_bm64_bn128_s4", "rows16_tiled_bm128_bn256_s3"]:
        Y = _gemm_bf16(gh, bits, packed, M, N, K, rows16[nm], 3)
        checked = 0
        for r in range(M):
            cols = np.nonzero(W16[big_k[r]] == 0.0)[0]
            exp = _f32_bf16_rne((small_v[r] * W16[small_k[r], cols]).astype(np.float32))
            nz = (exp & 0x7FFF) != 0                                   # +-0 compare equal
            assert np.array_equal(Y[r, cols][nz], exp[nz]), (nm, r, Es[r % len(Es)],
                                                             deltas[r % len(deltas)])
            assert np.all((Y[r, cols][~nz] & 0x7FFF) == 0), (nm, r)
            checked += len(cols)
        assert checked > 20 * M


@pytest.mark.parametrize("M,K,N,asym", [(1024, 8192, 10240, True), (48, 28672, 8192, False)])
def test_bf16_rows16_groups_of_64_full_size(gh, M, K, N, asym):
    """Groups of 64 rows with bf16 activations above 32 rows: fp16 rows on the tiled kernel
    (the skinny kernel is kept up to 32 rows)."""
    _, d, bits, vals = _case_bf16(M, K, N, asym, group=64)
    Y = _bf16_f32(_gemm_bf16(gh, bits, gh.repack(d, K, N, 64), M, N, K, group=64))
    assert np.all(np.isfinite(Y))
    rows, cols = gh.tile_samples(M, N)
    Yref, B = oracle.gemm_sampled(vals, d["Qp"], d["s"], d["Zp"], 64, rows, cols)
    ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, B, rel_fro=BF16_FRO)
    assert ok, info


@pytest.mark.parametrize("M,K,N,asym", [(1, 4096, 11008, False), (16, 4096, 11008, True),
                                        (32, 11008, 4096, False), (256, 8192, 10240, False),
                                        (1024, 28672, 8192, True), (192, 8192, 28672, False),
                                        (4096, 28672, 8192, False)])
def test_bf16_full_size(gh, M, K, N, asym):
    _, d, bits, vals = _case_bf16(M, K, N, asym)
    Y = _bf16_f32(_gemm_bf16(gh, bits, gh.repack(d, K, N), M, N, K))  # NaN-filled before
    assert np.all(np.isfinite(Y))
    rows, cols = gh.tile_samples(M, N)
    Yref, B = oracle.gemm_sampled(vals, d["Qp"], d["s"], d["Zp"], 128, rows, cols)
    ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, B, rel_fro=BF16_FRO)
    assert ok, info


@pytest.mark.parametrize("M,K,N,asym", [(5, 1152, 528, True), (33, 2048, 1040, False),
                                        (16, 4096, 11008, True)])
def test_bf16_groups_of_64(gh, M, K, N, asym):
    """bf16 activations with groups of 64 rows: activation sums, offsets and scales per
    64-row half; automatic plan and a spread of explicit variants and K splits."""
    _, d, bits, vals = _case_bf16(M, K, N, asym, group=64)
    packed = gh.repack(d, K, N, 64)
    Yref = oracle.gemm(vals, d["Qp"], d["s"], d["Zp"], 64)
    B = oracle.error_bound(vals, d["Qp"], d["s"], d["Zp"], 64)
    plans = [(-1, 0), (gh.variant_index("skinny_xr4_nt1_wk8_d4"), 3),
             (gh.variant_index("skinny_xr16_nt2_wk8_d2"), 1),
             (gh.variant_index("skinny_xr32_nt1_wk4_d2"), 2),
             (gh.variant_index("skinny_xr64_nt1_wk4_d2"), 1)]
    for v, splits in plans:
        if v >= 0 and N % (16 * int(gh.w4.w4a16_gemm_variant_name(v).split("_nt")[1].split("_")[0])):
            continue  # this variant's column tiles do not divide N
        Y = _bf16_f32(_gemm_bf16(gh, bits, packed, M, N, K, v, splits, group=64))
        ok, info = oracle.accept(Y, Yref, B, rel_fro=BF16_FRO)
        assert ok, (v, splits, info)


@pytest.mark.parametrize("asym", [False, True])
def test_bf16_groups_of_64_onehot_exact(gh, asym):
    """One-hot bf16 rows with groups of 64 select RNE_bf16((q - z) * s) bit for bit."""
    M, K, N = 16, 1024, 768
    _, d, _, _ = _case_bf16(M, K, N, asym, group=64)
    ks = [0, 1, 7, 8, 9, 63, 64, 127, 128, 255, 300, 511, 640, 777, 900, 1023]
    bits = np.zeros((M, K), np.uint16)
    bits[np.arange(M), ks] = 0x3F80  # 1.0
    W = oracle.dequant(d["Qp"], d["s"], d["Zp"], K, N, 64)
    exp = _f32_bf16_rne(W[ks].astype(np.float32))
    packed = gh.repack(d, K, N, 64)
    for nm, splits in [("skinny_xr16_nt1_wk8_d2", 1), ("skinny_xr16_nt4_wk4_d2", 3)]:
        Y = _gemm_bf16(gh, bits, packed, M, N, K, gh.variant_index(nm), splits, group=64)
        assert np.array_equal(Y, exp), nm


def test_caller_owned_workspace(gh):
    """w4a16_set_workspace: split-K (skinny) and stream-K (tiled) launches on a stream with a
    caller-owned buffer give the same bits as on a stream with a library-owned one, twice in
    a row (the counters come back to zero); a buffer too small for a plan is refused with
    an error instead of grown; NULL hands the stream back to the library."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    cases = [(8, 11008, 4096, gh.variant_index("skinny_xr8_nt1_wk8_d4"), 3),
             (300, 2048, 1040, gh.variant_index("tiled_bm128_bn256_s3"), 7)]
    prepared = []
    for (M, K, N, v, sp) in cases:
        _, d, X = _case(M, K, N, asym=True)
        prepared.append((M, K, N, v, sp, gh.dev(X), gh.repack(d, K, N)))
    ref = []
    for (M, K, N, v, sp, Xd, packed) in prepared:
        ref.append(gh.host(gh.gemm(Xd, packed, M, N, K, variant=v, splits=sp)).view(np.uint16).copy())
    st = torch.cuda.Stream()
    buf = torch.empty(w4.WS_COUNTER_BYTES + (8 << 20), dtype=torch.uint8, device="cuda")
    w4.w4a16_set_workspace(buf, buf.numel(), stream=st)
    try:
        for _ in range(2):
            with torch.cuda.stream(st):
                outs = [gh.gemm(Xd, packed, M, N, K, variant=v, splits=sp)
                        for (M, K, N, v, sp, Xd, packed) in prepared]
            torch.cuda.synchronize()
            for o, r in zip(outs, ref):
                assert np.array_equal(gh.host(o).view(np.uint16), r)
        small = torch.empty(w4.WS_COUNTER_BYTES + 256, dtype=torch.uint8, device="cuda")
        w4.w4a16_set_workspace(small, small.numel(), stream=st)
        M, K, N, v, sp, Xd, packed = prepared[1]
        with torch.cuda.stream(st), pytest.raises(w4.W4A16Error):
            gh.gemm(Xd, packed, M, N, K, variant=v, splits=sp)
        torch.cuda.synchronize()
    finally:
        w4.w4a16_set_workspace(None, 0, stream=st)
    with torch.cuda.stream(st):
        outs = [gh.gemm(Xd, packed, M, N, K, variant=v, splits=sp)
                for (M, K, N, v, sp, Xd, packed) in prepared]
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert np.array_equal(gh.host(o).view(np.uint16), r)


# ---- groups of more than 128 rows: 256, and one group spanning all of K ----------------
# The repacked layout stores one scale (and zero-point) row per 128-row block, a group of
# 256 or more rows once per block it spans, so every kernel and entry point sees the same
# format as for groups of 128; the repack's replication, the unpack's choice of copy and
# the oracle's group indexing are what these tests pin.
def _case_big(M, K, N, group, asym=False, seed=0):
    w = Workload(cfg=9, M=M, K=K, N=N, group=group, asym=asym)
    d = weights(w, seed=9000 + seed + K + N + group)
    X = activations(w, seed=9500 + seed + M)
    return w, d, X


BIG_GROUPS = [256, "K"]


def _g(group, K):
    return K if group == "K" else group


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("group", BIG_GROUPS)
def test_big_group_repack_layout_and_roundtrip(gh, group, asym):
    import torch
    import layout_model as lm
    import w4a16_mixed_precision_offline_amd as w4
    K, N = 1536, 528
    g = _g(group, K)
    _, d, _ = _case_big(1, K, N, g, asym)
    wp, sp, zp = gh.repack(d, K, N, g)
    assert np.array_equal(gh.host(wp).view(np.uint32), lm.repack_codes(d["Qp"], K, N))
    assert np.array_equal(gh.host(sp).view(np.uint16),
                          lm.repack_scales(d["s"], N, g // 128).view(np.uint16))
    if asym:
        assert np.array_equal(gh.host(zp).view(np.uint32), lm.repack_zeros(d["Zp"], N, g // 128))
    q = torch.zeros((K // 8, N), dtype=torch.int32, device="cuda")
    s = torch.zeros((K // g, N), dtype=torch.float16, device="cuda")
    z = torch.zeros((K // g, N // 8), dtype=torch.int32, device="cuda") if asym else None
    w4.w4a16_unpack(wp, sp, zp, q, s, z, K, N, g)
    assert np.array_equal(gh.host(q), d["Qp"])
    assert np.array_equal(gh.host(s).view(np.uint16), d["s"].view(np.uint16))
    if asym:
        assert np.array_equal(gh.host(z), d["Zp"])


@pytest.mark.parametrize("group", BIG_GROUPS)
@pytest.mark.parametrize("M,K,N,asym", [(5, 1536, 528, True), (33, 1024, 512, False),
                                        (300, 2048, 1040, True), (1, 512, 48, False)])
def test_big_group_every_variant(gh, group, M, K, N, asym):
    import w4a16_mixed_precision_offline_amd as w4
    g = _g(group, K)
    _, d, X = _case_big(M, K, N, g, asym)
    packed = gh.repack(d, K, N, g)
    Xd = gh.dev(X)
    Yref = oracle.gemm(X, d["Qp"], d["s"], d["Zp"], g)
    B = oracle.error_bound(X, d["Qp"], d["s"], d["Zp"], g)
    ran = 0
    for v in [-1] + list(range(w4.w4a16_gemm_variants())):
        name = w4.w4a16_gemm_variant_name(v) if v >= 0 else "auto"
        nt = 1 if not name.startswith("skinny") else int(name.split("_nt")[1].split("_")[0])
        if N % (16 * nt):
            continue
        for splits in ((0,) if v < 0 else (1, 3)):
            Y = gh.nan_filled(M, N)
            gh.gemm(Xd, packed, M, N, K, group=g, variant=v, splits=splits, Y=Y)
            ok, info = oracle.accept(gh.host(Y), Yref, B)
            assert ok, (group, name, splits, info)
            ran += 1
    assert ran > 1


@pytest.mark.parametrize("asym", [False, True])
@pytest.mark.parametrize("group", BIG_GROUPS)
def test_big_group_onehot_exact(gh, group, asym):
    """One-hot rows on both sides of every 128-row block boundary select RNE((q - z) * s)
    of their group, through the skinny paths (fp32 rescale and fp16-scaled weights) and
    the tiled kernel."""
    M, K, N = 16, 1024, 768
    g = _g(group, K)
    _, d, _ = _case_big(M, K, N, g, asym)
    ks = [0, 1, 127, 128, 129, 255, 256, 257, 383, 384, 511, 512, 640, 767, 768, 1023]
    X = np.zeros((M, K), np.float16)
    X[np.arange(M), ks] = 1.0
    W16 = oracle.dequant_fp16(d["Qp"], d["s"], d["Zp"], K, N, g)
    packed = gh.repack(d, K, N, g)
    names = ["skinny_xr16_nt2_wk8_d2", "skinny_xr16_nt4_wk4_d2", "tiled_bm128_bn256_s3",
             "tiled_bm16_bn256_s4"]
    for nm in names:
        for splits in (1, 3):
            Y = gh.host(gh.gemm(gh.dev(X), packed, M, N, K, group=g,
                                variant=gh.variant_index(nm), splits=splits))
            assert np.array_equal(Y.view(np.uint16), W16[ks].view(np.uint16)), (nm, splits)


@pytest.mark.parametrize("group", BIG_GROUPS)
@pytest.mark.parametrize("M,K,N,asym", [(16, 4096, 11008, True), (1024, 8192, 10240, False)])
def test_big_group_full_size(gh, group, M, K, N, asym):
    g = _g(group, K)
    _, d, X = _case_big(M, K, N, g, asym)
    Y = gh.host(gh.gemm(gh.dev(X), gh.repack(d, K, N, g), M, N, K, group=g,
                        Y=gh.nan_filled(M, N)))
    assert np.all(np.isfinite(Y))
    rows, cols = gh.tile_samples(M, N)
    Yref, B = oracle.gemm_sampled(X, d["Qp"], d["s"], d["Zp"], g, rows, cols)
    ok, info = oracle.accept(Y[np.ix_(rows, cols)], Yref, B)
    assert ok, info


@pytest.mark.parametrize("group", BIG_GROUPS)
@pytest.mark.parametrize("M,K,N,asym", [(5, 1536, 528, True), (300, 2048, 1040, False)])
def test_big_group_bf16_and_fp8_activations(gh, group, M, K, N, asym):
    """The bf16 and the fp8 (W4A8) entry points on the same repacked weights with a group
    of 256 rows or one group spanning K, automatic plans, against the oracle."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    from gen import activations_bf16, activations_fp8
    g = _g(group, K)
    w, d, _ = _case_big(M, K, N, g, asym)
    wp, sp, zp = gh.repack(d, K, N, g)
    bits, vals = activations_bf16(w, seed=9600 + M)
    Yb = torch.full((M, N), -1, dtype=torch.int16, device="cuda")
    w4.w4a16_gemm_bf16(gh.dev(bits.view(np.int16)), wp, sp, zp, Yb, M, N, K, g)
    ok, info = oracle.accept(_bf16_f32(gh.host(Yb).view(np.uint16)),
                             oracle.gemm(vals, d["Qp"], d["s"], d["Zp"], g),
                             oracle.error_bound(vals, d["Qp"], d["s"], d["Zp"], g), rel_fro=BF16_FRO)
    assert ok, ("bf16", info)
    X8, a = activations_fp8(w, seed=9700 + M)
    Y8 = gh.nan_filled(M, N)
    w4.w4a8_gemm(gh.dev(X8), gh.dev(a), wp, sp, zp, Y8, M, N, K, g)
    ok, info = oracle.accept(gh.host(Y8), oracle.gemm_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], g),
                             oracle.error_bound_w4a8(X8, a, d["Qp"], d["s"], d["Zp"], g))
    assert ok, ("fp8", info)
