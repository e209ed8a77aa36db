"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/w4a16.h declares, and rejects invalid arguments on the host before any
HIP call.  No compute entry point is ever called with arguments that would pass
validation (those tests live in the GPU suite)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")
LIB = os.path.join(ROOT, "w4a16_mixed_precision_offline_amd", "libw4a16.so")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(w4a(?:16|8)_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def raw():
    if not os.path.exists(LIB):
        pytest.fail("libw4a16.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("w4a16_repack", "w4a16_gemm", "w4a16_unpack", "w4a16_dequant",
              "w4a16_fp16_gemm", "w4a16_packed_bytes", "w4a16_strerror", "w4a8_gemm",
              "w4a8_gemm_plan"):
        assert n in names


def test_every_declared_symbol_is_exported(raw):
    for n in declared_functions():
        assert hasattr(raw, n), n


def test_binding_covers_every_declared_symbol():
    import w4a16_mixed_precision_offline_amd as w4
    for n in declared_functions():
        assert n in w4.EXPORTED and callable(getattr(w4, n)), n


def test_binding_constants_match_the_header():
    import w4a16_mixed_precision_offline_amd as w4
    text = open(HEADER).read()
    m = re.search(r"#define W4A16_NOALLOC_SCRATCH_BYTES \((\d+) \+ \((\d+)u << (\d+)\)\)", text)
    assert m, "W4A16_NOALLOC_SCRATCH_BYTES not found"
    a, b, c = (int(g) for g in m.groups())
    assert w4.NOALLOC_SCRATCH_BYTES == a + (b << c)


def test_queries(raw):
    raw.w4a16_strerror.restype = ctypes.c_char_p
    raw.w4a16_packed_bytes.restype = ctypes.c_size_t
    assert raw.w4a16_layout_version() == 1
    for code in range(0, -9, -1):
        assert raw.w4a16_strerror(code)
    assert b"unknown" in raw.w4a16_strerror(42)
    assert raw.w4a16_packed_bytes(4096, 4096, 128, 0) == 4096 * 4096 // 2
    assert raw.w4a16_packed_bytes(4096, 4096, 128, 1) == 2 * 32 * 4096
    assert raw.w4a16_packed_bytes(4096, 4096, 128, 2) == 32 * 4096 // 2
    assert raw.w4a16_packed_bytes(4096, 4096, 256, 1) == 2 * 32 * 4096   # one row per 128 K
    assert raw.w4a16_packed_bytes(4096, 4096, 256, 2) == 32 * 4096 // 2
    assert raw.w4a16_packed_bytes(4096, 4096, 128, 3) == 4096 * 4096 // 4
    assert raw.w4a16_packed_bytes(4096, 4096, 128, 4) == 4096 * 4096 // 8
    assert raw.w4a16_packed_bytes(4096, 4096, 128, 9) == 0
    assert raw.w4a16_packed_bytes(4096, 4104, 128, 0) == 0   # N % 16
    assert raw.w4a16_packed_bytes(4000, 4096, 128, 0) == 0   # K % group
    assert raw.w4a16_packed_bytes(4096, 4096, 32, 0) == 0    # group neither 64 nor 128j
    assert raw.w4a16_packed_bytes(4096, 4096, 192, 0) == 0
    # groups of 64 rows: two scale (and zero-point) rows per 128-row block; no 2:4 format
    assert raw.w4a16_packed_bytes(4096, 4096, 64, 0) == 4096 * 4096 // 2
    assert raw.w4a16_packed_bytes(4096, 4096, 64, 1) == 2 * 64 * 4096
    assert raw.w4a16_packed_bytes(4096, 4096, 64, 2) == 64 * 4096 // 2
    assert raw.w4a16_packed_bytes(4096, 4096, 64, 3) == 0
    assert raw.w4a16_packed_bytes(4096, 4096, 64, 5) == 0
    assert raw.w4a16_gemm_variants() >= 1


def test_describe_plans(raw):
    out = (ctypes.c_int * 4)()
    for (M, K, N) in [(1, 4096, 4096), (32, 4096, 11008), (16, 1024, 1024), (4096, 8192, 28672),
                      (48, 3072, 768)]:
        assert raw.w4a16_gemm_describe(M, N, K, 128, out) == 0
        assert 0 <= out[0] < raw.w4a16_gemm_variants()
        assert out[1] >= 1 and out[2] >= 1 and out[3] in (64, 128, 256, 512, 1024)
    # wide layers: three column tiles per wave where that fills the 256 compute units
    # better (N = 12288: 256 workgroups), else four (N = 11008: 172)
    raw.w4a16_gemm_variant_name.restype = ctypes.c_char_p
    for (N, name) in [(12288, b"skinny_xr16_nt3_wk4_d2"), (11008, b"skinny_xr16_nt4_wk4_d2")]:
        assert raw.w4a16_gemm_describe(16, N, 4096, 128, out) == 0
        assert raw.w4a16_gemm_variant_name(out[0]) == name
    # wide layers where four tiles per wave would leave under 160 workgroups: two, unless
    # K is long enough to split (K >= 12288: four tiles, K in slices)
    for (N, K, name) in [(5120, 8192, b"skinny_xr16_nt2_wk8_d2"), (8192, 8192, b"skinny_xr16_nt2_wk8_d2"),
                         (5120, 13824, b"skinny_xr16_nt4_wk4_d2"), (8192, 28672, b"skinny_xr16_nt4_wk4_d2")]:
        assert raw.w4a16_gemm_describe(16, N, K, 128, out) == 0
        assert raw.w4a16_gemm_variant_name(out[0]) == name
    # above 32 rows: the tiled kernel, except on layers under 32 Mi weights below 256 rows,
    # which take the skinny kernel in blocks of 16 or 32 rows
    for (M, N, K, name) in [(48, 13824, 5120, b"tiled_bm64_bn128_s4"), (48, 768, 3072, b"skinny_xr16_nt1_wk8_d2"),
                            (48, 28672, 8192, b"tiled_bm64_bn256_s3"),
                            (128, 768, 3072, b"skinny_xr32_nt1_wk4_d2"),
                            (128, 8192, 8192, b"tiled_bm128_bn128_s3"), (128, 8192, 28672, b"tiled_bm128_bn256_w8_s3"), (48, 2560, 2560, b"skinny_xr16_nt2_wk8_d2"),
                            (128, 4096, 4096, b"skinny_xr32_nt4_wk4_d2"), (32, 28672, 8192, b"skinny_xr32_nt4_wk4_d2")]:
        assert raw.w4a16_gemm_describe(M, N, K, 128, out) == 0
        assert raw.w4a16_gemm_variant_name(out[0]) == name, (M, N, K)
    assert raw.w4a16_gemm_describe(0, 4096, 4096, 128, out) == -2
    assert raw.w4a16_gemm_describe(1, 4096, 4096, 128, None) == -1


A = 256        # a fake, aligned, non-null address: only ever used where validation fails
MIS = 258      # misaligned


def gemm(raw, X=A, wp=A, sp=A, zp=None, Y=A, M=16, N=1024, K=1024, g=128):
    f = raw.w4a16_gemm
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    return f(X, wp, sp, zp, Y, M, N, K, g, None)


def test_gemm_validation(raw):
    assert gemm(raw, X=None) == -1
    assert gemm(raw, wp=None) == -1
    assert gemm(raw, sp=None) == -1
    assert gemm(raw, Y=None) == -1
    assert gemm(raw, M=0) == -2
    assert gemm(raw, N=1000) == -2       # N % 16
    assert gemm(raw, K=1000) == -2       # K % 128
    assert gemm(raw, g=32) == -2         # group neither 64 nor a multiple of 128
    assert gemm(raw, g=192) == -2
    assert gemm(raw, g=384) == -2        # K % group
    assert gemm(raw, K=-128) == -2
    assert gemm(raw, X=MIS) == -3
    assert gemm(raw, Y=MIS) == -3
    assert gemm(raw, zp=MIS) == -3


def test_repack_validation(raw):
    f = raw.w4a16_repack
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert f(None, A, None, A, A, None, 1024, 1024, 128, None) == -1
    assert f(A, A, A, A, A, None, 1024, 1024, 128, None) == -1   # z without zp
    assert f(A, A, None, A, A, A, 1024, 1024, 128, None) == -1   # zp without z
    assert f(A, A, None, A, A, None, 1024, 1000, 128, None) == -2
    assert f(A, A, None, A, A, None, 1024, 1024, 96, None) == -2
    assert f(MIS, A, None, A, A, None, 1024, 1024, 128, None) == -3
    g = raw.w4a16_unpack
    g.argtypes = f.argtypes
    assert g(A, A, None, None, A, None, 1024, 1024, 128, None) == -1
    assert g(A, A, None, A, A, None, 0, 1024, 128, None) == -2


def test_workspace_bytes(raw):
    f = raw.w4a16_workspace_bytes
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int] * 3
    assert f(0, 4096, 4096) == 0 and f(16, 4000, 4096) == 0 and f(16, 4096, 100) == 0
    # a wide decode layer runs without cross-workgroup reduction
    assert f(1, 12288, 4096) == 0
    # 8192 x 10240 at M = 256: 160 tiles of 128 x 128 on 256 workgroups, all striped:
    # two fp32 partial tiles per workgroup
    assert f(256, 10240, 8192) >= 2 * 256 * 128 * 128 * 4
    # M = 4096 on the same layer: 14 (fp16 tiles: 28) whole rounds of tiles, no stripes;
    # what remains is w4a16_gemm_bf16's fp16 rows (M*K*2 bytes) and fp32 row scales
    assert f(4096, 28672, 8192) == 4096 * 4 + 4096 * 8192 * 2


def test_fp16_plan_validation(raw):
    f = raw.w4a16_fp16_gemm_plan
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    raw.w4a16_fp16_gemm_variant_name.restype = ctypes.c_char_p
    n = raw.w4a16_fp16_gemm_variants()
    names = [raw.w4a16_fp16_gemm_variant_name(v) for v in range(n)]
    assert all(names) and raw.w4a16_fp16_gemm_variant_name(n) is None
    # the skinny variants (numbered as in w4a16_gemm_variants) plus the fp16 tiled ones
    raw.w4a16_gemm_variant_name.restype = ctypes.c_char_p
    skinny = [raw.w4a16_gemm_variant_name(v) for v in range(raw.w4a16_gemm_variants())
              if not raw.w4a16_gemm_variant_name(v).startswith(b"tiled")]
    assert names[:len(skinny)] == skinny
    assert len(names) - len(skinny) >= 2
    assert all(nm.startswith(b"tiled_f16") for nm in names[len(skinny):])
    assert f(None, A, A, 1, 16, 128, -1, 0, None) == -1
    assert f(A, A, A, 1, 16, 100, -1, 0, None) == -2
    assert f(A, A, A, 1, 16, 128, n, 0, None) == -8
    assert f(A, A, A, 1, 16, 128, -2, 0, None) == -8
    assert f(A, A, A, 1, 16, 128, 0, -1, None) == -8
    assert f(A, MIS, A, 1, 16, 128, -1, 0, None) == -3


def test_probe_validation(raw):
    f = raw.w4a16_probe_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 16, A, None) == -1
    assert f(A, 16, None, None) == -1
    assert f(A, 0, A, None) == -2
    assert f(A, 24, A, None) == -2
    assert f(MIS, 16, A, None) == -3
    g = raw.w4a16_probe_mfma
    g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert g(1, 1, None, None) == -1
    assert g(0, 1, A, None) == -8 and g(65537, 1, A, None) == -8 and g(1, 0, A, None) == -8
    h = raw.w4a16_probe_mfma_flops
    h.restype = ctypes.c_double
    h.argtypes = [ctypes.c_int, ctypes.c_int]
    assert h(256, 10) == 256 * 4 * 10 * 4 * 2 * 32 * 32 * 16
    assert h(0, 10) == 0.0


def test_bf16_validation(raw):
    f = raw.w4a16_gemm_bf16_plan
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    assert f(None, A, A, None, A, 16, 1024, 1024, 128, -1, 0, None) == -1
    assert f(A, A, A, None, A, 16, 1024, 1024, 192, -1, 0, None) == -2  # not 64 nor 128j
    assert f(A, A, A, None, A, 16, 1000, 1024, 128, -1, 0, None) == -2
    raw.w4a16_gemm_variant_name.restype = ctypes.c_char_p
    nskinny = sum(1 for v in range(raw.w4a16_gemm_variants())
                  if not raw.w4a16_gemm_variant_name(v).startswith(b"tiled"))
    total = raw.w4a16_gemm_variants()
    w8 = [v for v in range(total) if b"_w8_" in raw.w4a16_gemm_variant_name(v)]
    assert w8
    # tiled variants take bf16 activations (four-wave tiles: without a GPU the plan passes
    # and the missing device is reported; with one this call would launch on the fake
    # pointers, so it only runs where there is none), not the eight-wave ones, and not with
    # groups of 64 rows
    import os
    if not os.path.exists("/dev/kfd"):
        assert f(A, A, A, None, A, 256, 1024, 1024, 128, nskinny, 0, None) == -4
    assert f(A, A, A, None, A, 256, 1024, 1024, 128, w8[0], 0, None) == -8
    assert f(A, A, A, None, A, 256, 1024, 1024, 64, nskinny, 0, None) == -8
    # then the fp16 tiled variants on rows rewritten in fp16, every group size included
    raw.w4a16_gemm_bf16_variants.restype = ctypes.c_int
    raw.w4a16_gemm_bf16_variant_name.restype = ctypes.c_char_p
    nb = raw.w4a16_gemm_bf16_variants()
    assert nb == total + (total - nskinny)
    names = [raw.w4a16_gemm_bf16_variant_name(v) for v in range(nb)]
    assert names[:total] == [raw.w4a16_gemm_variant_name(v) for v in range(total)]
    assert names[total:] == [b"rows16_" + raw.w4a16_gemm_variant_name(v)
                             for v in range(nskinny, total)]
    assert raw.w4a16_gemm_bf16_variant_name(nb) is None
    assert raw.w4a16_gemm_bf16_variant_name(-1) is None
    if not os.path.exists("/dev/kfd"):
        assert f(A, A, A, None, A, 256, 1024, 1024, 64, total, 0, None) == -4
    assert f(A, A, A, None, A, 16, 1024, 1024, 128, nb, 0, None) == -8
    assert f(A, A, A, None, A, 16, 1024, 1024, 128, -2, 0, None) == -8


def test_set_workspace_validation(raw):
    f = raw.w4a16_set_workspace
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(A + 16, 1 << 20, None) == -3          # not 256-byte aligned
    assert f(A, 65536, None) == -6                 # no room past the counter prefix


def test_w4a8_validation(raw):
    f = raw.w4a8_gemm_plan
    f.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    assert f(None, None, A, A, None, A, 16, 1024, 1024, 128, -1, 0, None) == -1
    assert f(A, None, A, None, None, A, 16, 1024, 1024, 128, -1, 0, None) == -1  # no scales
    assert f(A, None, A, A, None, A, 16, 1024, 1024, 192, -1, 0, None) == -2  # not 64 nor 128j
    assert f(A, None, A, A, None, A, 16, 1000, 1024, 128, -1, 0, None) == -2
    assert f(A, None, A, A, None, A, 0, 1024, 1024, 128, -1, 0, None) == -2
    assert f(MIS, None, A, A, None, A, 16, 1024, 1024, 128, -1, 0, None) == -3
    assert f(A, A + 2, A, A, None, A, 16, 1024, 1024, 128, -1, 0, None) == -3  # row scales
    raw.w4a16_gemm_variant_name.restype = ctypes.c_char_p
    nskinny = sum(1 for v in range(raw.w4a16_gemm_variants())
                  if not raw.w4a16_gemm_variant_name(v).startswith(b"tiled"))
    nall = raw.w4a16_gemm_variants()
    assert nskinny < nall
    # numbered like w4a16_gemm_bf16_plan: skinny, fp8 tiled, then fp16 tiled on rewritten
    # rows (those pass the host checks: without a GPU the missing device is reported; with
    # one this call would launch on the fake pointers, so it only runs where there is none)
    nb = raw.w4a16_gemm_bf16_variants()
    assert nb == nall + (nall - nskinny)
    import os
    if not os.path.exists("/dev/kfd"):
        assert f(A, None, A, A, None, A, 64, 1024, 1024, 64, nall, 0, None) == -4
    assert f(A, None, A, A, None, A, 16, 1024, 1024, 128, nb, 0, None) == -8  # out of range
    assert f(A, None, A, A, None, A, 16, 1024, 1024, 128, -1, -1, None) == -8
    g = raw.w4a8_gemm
    g.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    assert g(A, None, A, A, None, None, 16, 1024, 1024, 128, None) == -1   # no output
    assert g(A, None, A, A, None, A, 16, 1024, 1000, 128, None) == -2


def test_mxfp4_validation(raw):
    """MXFP4 entry points: every host-side check returns its code before any HIP call."""
    f = raw.w4a8_mx_gemm_plan
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 5 + [ctypes.c_void_p]
    assert f(None, None, A, A, A, 16, 1024, 1024, -1, 0, None) == -1
    assert f(A, None, A, None, A, 16, 1024, 1024, -1, 0, None) == -1   # no scales
    assert f(A, None, A, A, None, 16, 1024, 1024, -1, 0, None) == -1   # no output
    assert f(A, None, A, A, A, 16, 1000, 1024, -1, 0, None) == -2      # N % 16
    assert f(A, None, A, A, A, 16, 1024, 1000, -1, 0, None) == -2      # K % 128
    assert f(A, None, A, A, A, 0, 1024, 1024, -1, 0, None) == -2       # M = 0
    assert f(MIS, None, A, A, A, 16, 1024, 1024, -1, 0, None) == -3
    assert f(A, A + 2, A, A, A, 16, 1024, 1024, -1, 0, None) == -3     # row scales
    nv = raw.w4a8_mx_variants()
    assert f(A, None, A, A, A, 16, 1024, 1024, nv, 0, None) == -8      # out of range
    assert f(A, None, A, A, A, 16, 1024, 1024, -2, 0, None) == -8
    assert f(A, None, A, A, A, 16, 1024, 1024, 0, -1, None) == -8      # negative grid
    assert f(A, None, A, A, A, 33, 1024, 1024, nv - 1, 0, None) == -8  # decode kernel, M > 32
    r = raw.w4a8_mx_repack
    r.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 2 + [ctypes.c_void_p]
    assert r(None, A, A, A, 1024, 1024, None) == -1
    assert r(A, None, A, A, 1024, 1024, None) == -1
    assert r(A, A, A, A, 1000, 1024, None) == -2
    assert r(A, A, A, A, 1024, 1000, None) == -2
    assert r(A, A, A, A, 1 << 20, 1 << 14, None) == -2                 # K*N/8 >= 2^31
    assert r(MIS, A, A, A, 1024, 1024, None) == -3


def test_baseline_validation(raw):
    f = raw.w4a16_fp16_gemm
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert f(None, A, A, 1, 16, 128, None) == -1
    assert f(A, A, A, 1, 16, 100, None) == -2
    assert f(A, A, A, 1, 15, 128, None) == -2
    assert f(A, MIS, A, 1, 16, 128, None) == -3
    d = raw.w4a16_dequant
    d.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert d(A, A, None, None, 128, 16, 128, None) == -1
    assert d(A, A, None, A, 100, 16, 128, None) == -2


def test_plan_validation(raw):
    f = raw.w4a16_gemm_plan
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    assert f(A, A, A, None, A, 16, 1024, 1024, 128, 10 ** 6, 0, None) == -8
    assert f(A, A, A, None, A, 16, 1024, 1024, 128, -2, 0, None) == -8
    assert f(A, A, A, None, A, 16, 1024, 1024, 128, -1, -1, None) == -8
    assert f(None, A, A, None, A, 16, 1024, 1024, 128, -1, 0, None) == -1


def test_sparse_validation(raw):
    f = raw.w4a16_sparse24_gemm
    f.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    assert f(A, A, None, A, A, 16, 1024, 1024, 128, None) == -1   # no positions
    assert f(A, A, A, A, A, 0, 1024, 1024, 128, None) == -2
    assert f(A, A, MIS, A, A, 16, 1024, 1024, 128, None) == -3
    r = raw.w4a16_sparse24_repack
    r.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert r(A, A, A, None, A, 1024, 1024, 128, None) == -1
    assert r(A, A, A, A, A, 1000, 1024, 128, None) == -2
    u = raw.w4a16_sparse24_unpack
    u.argtypes = r.argtypes
    assert u(A, A, A, None, A, 1024, 1024, 128, None) == -1
    p = raw.w4a16_sparse24_gemm_plan
    p.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [ctypes.c_void_p]
    assert p(A, A, A, A, A, 16, 1024, 1024, 128, 999, 0, None) == -8


def test_shapes_past_32_bit_descriptors_are_rejected_on_the_host(raw):
    """K = 2^25, N = 16 passes the weight-shape rules (K*N/8 = 2^26 words).  At M = 128 the
    tiled kernel's 128-row tiles and the skinny kernel's 32-row blocks of X span 2^33 and
    2^31 bytes: neither kernel's 32-bit buffer descriptors can address them, so the plan
    query and the GEMM itself must return W4A16_ERR_SHAPE (before any device call; the
    pointers below are never dereferenced).  At M = 64 (16-row blocks: 2^30 bytes) the
    skinny kernel serves the shape."""
    out = (ctypes.c_int * 4)()
    K, N = 1 << 25, 16
    assert raw.w4a16_gemm_describe(128, N, K, 128, out) == -2
    assert raw.w4a16_gemm_describe(64, N, K, 128, out) == 0
    assert raw.w4a16_gemm_describe(1, N, K, 128, out) == 0     # 4 rows: 2^28 bytes, fine
    p = ctypes.c_void_p(1 << 20)  # 16-byte aligned, never touched
    fn = raw.w4a16_gemm
    fn.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 4 + [ctypes.c_void_p]
    assert fn(p, p, p, None, p, 128, N, K, 128, None) == -2
    # groups of 64 rows run the skinny kernel at every M: the same guard applies
    assert raw.w4a16_gemm_describe(128, N, K, 64, out) == -2
    # the fp16 baseline: one workgroup's weight rows (16 columns x K fp16) past 2 GiB
    fp = raw.w4a16_fp16_gemm
    fp.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 3 + [ctypes.c_void_p]
    assert fp(p, p, p, 1, 16, 1 << 26, None) == -2


def test_binding_refuses_a_probe_read_past_a_tensor():
    """The streaming-read probe cannot see its buffer's size; the binding refuses, on the
    host, a byte count larger than the tensor it is given (nothing reaches the library)."""
    import torch
    import w4a16_mixed_precision_offline_amd as w4
    buf = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        w4.w4a16_probe_read(buf, 32, buf)
