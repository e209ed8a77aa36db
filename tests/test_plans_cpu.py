"""The automatic plans the measurements chose (host-only queries of the C ABI, no GPU):
which kernel and variant each workload shape gets, and the workspace the plans report."""
import pytest

w4 = pytest.importorskip("w4a16_mixed_precision_offline_amd")


def plan(M, N, K, group=128):
    d = w4.w4a16_gemm_describe(M, N, K, group)
    return d["name"], d["splits"]


@pytest.mark.parametrize("M,K,N,name", [
    # decode sweep: eight waves with four k-blocks in flight for 1-4 rows on narrow layers
    (1, 4096, 4096, "skinny_xr4_nt1_wk8_d4"), (4, 11008, 4096, "skinny_xr4_nt1_wk8_d4"),
    # wide layers at 1-2 rows: eight waves, two k-blocks in flight
    (1, 4096, 12288, "skinny_xr4_nt1_wk8_d2"), (2, 4096, 11008, "skinny_xr4_nt1_wk8_d2"),
    # four waves for eight rows on 4096 x 4096
    (8, 4096, 4096, "skinny_xr8_nt1_wk4_d4"),
    # three column tiles per wave where that fills the 256 compute units (N = 12288)
    (16, 4096, 12288, "skinny_xr16_nt3_wk4_d2"), (32, 4096, 12288, "skinny_xr32_nt3_wk4_d2"),
    # narrow layers at 17-32 rows: two 16-row blocks
    (32, 4096, 4096, "skinny_xr16_nt2_wk8_d2"), (20, 11008, 4096, "skinny_xr16_nt2_wk8_d2"),
    # above 32 rows on large layers: the tiled kernel, 64-row tiles up to 64 rows ...
    (48, 8192, 28672, "tiled_bm64_bn256_s3"), (64, 28672, 8192, "tiled_bm64_bn256_s3"),
    # ... 64 x 128 tiles on layers up to 128 Mi weights
    (48, 5120, 13824, "tiled_bm64_bn128_s4"), (64, 8192, 10240, "tiled_bm64_bn128_s4"),
    (48, 13824, 5120, "tiled_bm64_bn128_s4"),
    # ... 128-row tiles above, except where they would pad M by more than an eighth on
    # layers under 128 Mi weights up to 384 rows; on larger layers with eight waves
    (128, 8192, 28672, "tiled_bm128_bn256_w8_s3"), (192, 8192, 28672, "tiled_bm128_bn256_w8_s3"),
    (256, 28672, 8192, "tiled_bm128_bn256_w8_s3"), (192, 8192, 10240, "tiled_bm64_bn256_s3"),
    (320, 8192, 10240, "tiled_bm64_bn256_s3"), (448, 8192, 10240, "tiled_bm128_bn256_s3"),
    (448, 8192, 28672, "tiled_bm128_bn512_w8_s2"),
    # from a full round of 128 x 256 tiles on (where the 128 x 512 ones below do not fit
    # the chip in whole rounds): the same tiles with eight waves
    (1024, 8192, 10240, "tiled_bm128_bn256_w8_s3"), (1024, 28672, 8192, "tiled_bm128_bn256_w8_s3"),
    (2048, 8192, 10240, "tiled_bm128_bn256_w8_s3"),
    # eight-wave 128 x 512 tiles from two rounds of them on the 256 compute units on, or
    # in whole rounds of 224-256 workgroups
    (1024, 8192, 28672, "tiled_bm128_bn512_w8_s2"),
    (4096, 8192, 28672, "tiled_bm128_bn512_w8_s2"), (4096, 28672, 8192, "tiled_bm128_bn512_w8_s2"),
    (4096, 8192, 10240, "tiled_bm128_bn512_w8_s2"), (2048, 8192, 28672, "tiled_bm128_bn512_w8_s2"),
    (2048, 28672, 8192, "tiled_bm128_bn512_w8_s2"),
    # layers up to 128 Mi weights at 65-256 rows: 128 x 128 tiles
    (128, 5120, 13824, "tiled_bm128_bn128_s3"), (256, 8192, 10240, "tiled_bm128_bn128_s3"),
    # layers under 32 Mi weights stay on the skinny kernel at 33-255 rows, in blocks of 16
    # rows (up to 64) or 32, with the most column tiles per wave that keep 128 workgroups
    (48, 2560, 2560, "skinny_xr16_nt2_wk8_d2"), (128, 2560, 2560, "skinny_xr32_nt4_wk4_d2"),
    (48, 1024, 1024, "skinny_xr16_nt1_wk8_d2"), (128, 3072, 768, "skinny_xr32_nt1_wk4_d2"),
    (128, 4096, 4096, "skinny_xr32_nt4_wk4_d2"),
    # fewer than 128 column tiles: up to 16 rows in blocks of 4; two k-blocks in flight
    # when each wave has fewer than four
    (16, 3072, 768, "skinny_xr4_nt1_wk8_d2"), (1, 1024, 1024, "skinny_xr4_nt1_wk8_d2"),
    (1, 2560, 2560, "skinny_xr4_nt1_wk8_d2"),
])
def test_automatic_plans(M, K, N, name):
    assert plan(M, N, K)[0] == name


def test_eight_wave_tiles_take_whole_rounds_where_the_tile_count_allows():
    # 8 x 56 = 448 tiles: two rounds of 224 workgroups, no stream-K stripes; 32 x 56 = 1792:
    # seven rounds of 256; 32 x 20 = 640 tiles divide by nothing in 224..256: stream-K on 256
    # (the workspace query is the largest over the weight formats, so it is not checked
    # for the data-parallel case)
    assert w4.w4a16_gemm_describe(1024, 28672, 8192, 128)["workgroups"] == 224
    assert w4.w4a16_gemm_describe(4096, 28672, 8192, 128)["workgroups"] == 256
    assert w4.w4a16_gemm_describe(4096, 10240, 8192, 128)["workgroups"] == 256
    # 200-255 tiles of any variant: one round, one workgroup per tile
    assert w4.w4a16_gemm_describe(256, 28672, 8192, 128)["workgroups"] == 224
    assert w4.w4a16_gemm_describe(256, 13824, 5120, 128)["workgroups"] == 216
    assert w4.w4a16_gemm_describe(256, 10240, 8192, 128)["workgroups"] == 256
    assert w4.w4a16_workspace_bytes(4096, 10240, 8192) > 0


@pytest.mark.parametrize("M,K,N,name,splits", [
    # long K on layers with fewer than 160 blocks of 64 columns: four column tiles per
    # wave and K cut into slices that keep one round of workgroups (128 x 2, 80 x 3)
    (16, 28672, 8192, "skinny_xr16_nt4_wk4_d2", 2),
    (32, 28672, 8192, "skinny_xr32_nt4_wk4_d2", 2), (16, 13824, 5120, "skinny_xr16_nt4_wk4_d2", 3),
    (8, 13824, 5120, "skinny_xr8_nt4_wk4_d2", 3),
    # at 8 rows on N = 8192 two tiles per wave already fill the chip: no split
    (8, 28672, 8192, "skinny_xr8_nt2_wk8_d4", 1),
    # K = 8192 keeps two tiles per wave over the whole K; one to four rows are unchanged
    (16, 8192, 8192, "skinny_xr16_nt2_wk8_d2", 1), (1, 28672, 8192, "skinny_xr4_nt1_wk8_d2", 1),
])
def test_long_k_decode_plans_split_k(M, K, N, name, splits):
    assert plan(M, N, K) == (name, splits)


def test_k_split_only_where_workgroups_leave_most_of_the_chip_idle():
    # 4096 x 4096 at M = 1: 256 column tiles, no split; 3072 x 768 at M = 1: 48 workgroups,
    # no split either (the hand-off costs more); 4096 x 256: 16 workgroups, split
    assert plan(1, 4096, 4096)[1] == 1
    assert plan(1, 768, 3072)[1] == 1
    name, splits = plan(1, 256, 4096)
    assert name.startswith("skinny") and splits > 1


def test_2to4_plans_on_large_layers_need_workspace():
    # 32 rows: the 32-row tiles' stream-K pieces (16 rows: the 2:4 skinny plan reduces
    # inside its workgroups; the dense plans' needs are covered by the query too)
    assert w4.w4a16_workspace_bytes(32, 28672, 8192) > 0


def test_workspace_query_covers_the_split_plans():
    assert w4.w4a16_workspace_bytes(1, 4096, 4096) == 0          # no reduction across workgroups
    assert w4.w4a16_workspace_bytes(1, 256, 4096) > 0            # K split
    assert w4.w4a16_workspace_bytes(256, 10240, 8192) > 0        # stream-K pieces
    assert w4.w4a16_workspace_bytes(0, 4096, 4096) == 0          # invalid shape


def test_mxfp4_variant_table():
    """The MXFP4 entry points number the tiled variants first (the order of
    w4a16_gemm_variants) and then the three decode kernels."""
    import w4a16_mixed_precision_offline_amd as w4
    names = [w4.w4a8_mx_variant_name(v) for v in range(w4.w4a8_mx_variants())]
    tiled = [w4.w4a16_gemm_variant_name(v) for v in range(w4.w4a16_gemm_variants())
             if w4.w4a16_gemm_variant_name(v).startswith("tiled_")]
    assert names == tiled + ["mx_decode_nt1", "mx_decode_nt2", "mx_decode_nt4"]
    assert w4.w4a8_mx_variant_name(len(names)) is None
    assert w4.w4a8_mx_variant_name(-1) is None


def test_workspace_query_covers_the_fp8_and_mxfp4_plans():
    """At 17-32 rows on a 28672 x 8192 layer w4a16_gemm runs on the skinny kernel, while
    w4a8_mx_gemm keeps the 32-row tiled tile, whose 32 tiles are all cut into stream-K
    pieces over 256 workgroups: two 32 x 256 fp32 pieces per workgroup."""
    need = 2 * 256 * 32 * 256 * 4
    assert w4.w4a16_workspace_bytes(24, 8192, 28672) >= need
    # the decode kernel (M <= 16) reduces inside its workgroups only
    assert w4.w4a16_workspace_bytes(16, 28672, 8192) < need


def test_short_k_whole_piece_grids():
    """Four-wave 128 x 128 tiles on short K (at most 32 k-blocks) take whole pieces when
    they fill 160-199 compute units; longer K keeps the stream-K stripes."""
    d = w4.w4a16_gemm_describe(128, 12288, 4096, 128)       # 96 tiles, two pieces each
    assert d["name"] == "tiled_bm128_bn128_s3" and d["workgroups"] == 192
    d = w4.w4a16_gemm_describe(256, 12288, 4096, 128)       # 192 tiles, whole K
    assert d["name"] == "tiled_bm128_bn128_s3" and d["workgroups"] == 192
    d = w4.w4a16_gemm_describe(256, 11008, 4096, 64)        # groups of 64 too
    assert d["name"] == "tiled_bm128_bn128_s3" and d["workgroups"] == 172
    d = w4.w4a16_gemm_describe(256, 10240, 8192, 128)       # 64 k-blocks: stripes
    assert d["name"] == "tiled_bm128_bn128_s3" and d["workgroups"] == 256
