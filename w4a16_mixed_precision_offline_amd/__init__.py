"""Python binding of libw4a16 (MI355X / gfx950 W4A16 GEMM).

Argument marshalling only: every function below forwards to the C entry point of
the same name in libw4a16.so (declared in include/w4a16.h) and raises
W4A16Error on a non-zero return code.  Buffers may be torch tensors (their
data_ptr() is passed) or raw integer device addresses; `stream` defaults to
torch's current stream.  Every step of the computation runs in the HIP kernels;
there is no fallback path.  Importing fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(or python -m w4a16_mixed_precision_offline_amd.build_lib)")
# One HIP runtime per process.  torch's ROCm build ships its own libamdhip64 with the same
# soname as the system one this library links against: loaded after torch, the library
# binds to the runtime torch already holds; loaded before it, the process ends up with two
# runtimes and this library's finds no usable device.  So torch, when present, goes first.
try:
    import torch  # noqa: F401
except ImportError:
    pass
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t

_SIGS = {
    "w4a16_layout_version": (_I, []),
    "w4a16_strerror": (ctypes.c_char_p, [_I]),
    "w4a16_packed_bytes": (_SZ, [_I, _I, _I, _I]),
    "w4a16_repack": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "w4a16_unpack": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "w4a16_gemm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "w4a16_gemm_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "w4a16_gemm_plan": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "w4a16_gemm_variants": (_I, []),
    "w4a16_gemm_variant_name": (ctypes.c_char_p, [_I]),
    "w4a16_gemm_describe": (_I, [_I, _I, _I, _I, ctypes.POINTER(_I)]),
    "w4a16_workspace_bytes": (_SZ, [_I, _I, _I]),
    "w4a16_dequant": (_I, [_P, _P, _P, _P, _I, _I, _I, _P]),
    "w4a16_fp16_gemm": (_I, [_P, _P, _P, _I, _I, _I, _P]),
    "w4a16_fp16_gemm_plan": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "w4a16_fp16_gemm_variants": (_I, []),
    "w4a16_fp16_gemm_variant_name": (ctypes.c_char_p, [_I]),
    "w4a16_sparse24_repack": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "w4a16_sparse24_unpack": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "w4a16_sparse24_gemm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "w4a16_sparse24_gemm_plan": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "w4a16_gemm_bf16": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "w4a16_gemm_bf16_plan": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "w4a16_gemm_bf16_variants": (_I, []),
    "w4a16_gemm_bf16_variant_name": (ctypes.c_char_p, [_I]),
    "w4a8_gemm": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "w4a16_set_workspace": (_I, [_P, ctypes.c_size_t, _P]),
    "w4a8_gemm_plan": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P]),
    "w4a8_mx_repack": (_I, [_P, _P, _P, _P, _I, _I, _P]),
    "w4a8_mx_gemm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "w4a8_mx_gemm_plan": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "w4a8_mx_variants": (_I, []),
    "w4a8_mx_variant_name": (ctypes.c_char_p, [_I]),
    "w4a16_probe_read": (_I, [_P, _SZ, _P, _P]),
    "w4a16_probe_mfma": (_I, [_I, _I, _P, _P]),
    "w4a16_probe_mfma_flops": (ctypes.c_double, [_I, _I]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)

# buffer selectors of w4a16_packed_bytes
BUF_W, BUF_S, BUF_Z, BUF_SPARSE_V, BUF_SPARSE_I, BUF_SPARSE_S = range(6)


class W4A16Error(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {code} ({w4a16_strerror(code)})")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, code):
    if code != 0:
        raise W4A16Error(fn, code)


# ---- queries -----------------------------------------------------------------
def w4a16_layout_version() -> int:
    return _lib.w4a16_layout_version()


def w4a16_strerror(code: int) -> str:
    return _lib.w4a16_strerror(code).decode()


def w4a16_packed_bytes(K: int, N: int, group: int, which: int) -> int:
    return _lib.w4a16_packed_bytes(K, N, group, which)


def w4a16_gemm_variants() -> int:
    return _lib.w4a16_gemm_variants()


def w4a16_gemm_variant_name(v: int):
    r = _lib.w4a16_gemm_variant_name(v)
    return None if r is None else r.decode()


def w4a16_fp16_gemm_variants() -> int:
    return _lib.w4a16_fp16_gemm_variants()


def w4a16_fp16_gemm_variant_name(v: int):
    r = _lib.w4a16_fp16_gemm_variant_name(v)
    return None if r is None else r.decode()


def w4a16_workspace_bytes(M: int, N: int, K: int) -> int:
    return _lib.w4a16_workspace_bytes(M, N, K)


def w4a16_gemm_describe(M: int, N: int, K: int, group: int) -> dict:
    out = (_I * 4)()
    _check("w4a16_gemm_describe", _lib.w4a16_gemm_describe(M, N, K, group, out))
    return dict(variant=out[0], name=w4a16_gemm_variant_name(out[0]), splits=out[1],
                workgroups=out[2], threads=out[3])


# ---- compute entry points ------------------------------------------------------
def w4a16_repack(q, s, z, wp, sp, zp, K, N, group, stream=None):
    _check("w4a16_repack", _lib.w4a16_repack(_ptr(q), _ptr(s), _ptr(z), _ptr(wp), _ptr(sp),
                                             _ptr(zp), K, N, group, _stream(stream)))


def w4a16_unpack(wp, sp, zp, q, s, z, K, N, group, stream=None):
    _check("w4a16_unpack", _lib.w4a16_unpack(_ptr(wp), _ptr(sp), _ptr(zp), _ptr(q), _ptr(s),
                                             _ptr(z), K, N, group, _stream(stream)))


def w4a16_gemm(X, wp, sp, zp, Y, M, N, K, group, stream=None):
    _check("w4a16_gemm", _lib.w4a16_gemm(_ptr(X), _ptr(wp), _ptr(sp), _ptr(zp), _ptr(Y),
                                         M, N, K, group, _stream(stream)))


def w4a16_gemm_noalloc(X, wp, sp, zp, Y, M, N, K, group, stream=None):
    _check("w4a16_gemm_noalloc", _lib.w4a16_gemm_noalloc(_ptr(X), _ptr(wp), _ptr(sp), _ptr(zp),
                                                         _ptr(Y), M, N, K, group, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 65536 + (128 << 20)  # W4A16_NOALLOC_SCRATCH_BYTES


def w4a16_gemm_plan(X, wp, sp, zp, Y, M, N, K, group, variant=-1, splits=0, stream=None):
    _check("w4a16_gemm_plan", _lib.w4a16_gemm_plan(_ptr(X), _ptr(wp), _ptr(sp), _ptr(zp),
                                                   _ptr(Y), M, N, K, group, variant, splits,
                                                   _stream(stream)))


def w4a16_dequant(q, s, z, Wt, K, N, group, stream=None):
    _check("w4a16_dequant", _lib.w4a16_dequant(_ptr(q), _ptr(s), _ptr(z), _ptr(Wt), K, N,
                                               group, _stream(stream)))


def w4a16_fp16_gemm(X, Wt, Y, M, N, K, stream=None):
    _check("w4a16_fp16_gemm", _lib.w4a16_fp16_gemm(_ptr(X), _ptr(Wt), _ptr(Y), M, N, K,
                                                   _stream(stream)))


def w4a16_fp16_gemm_plan(X, Wt, Y, M, N, K, variant=-1, splits=0, stream=None):
    _check("w4a16_fp16_gemm_plan", _lib.w4a16_fp16_gemm_plan(
        _ptr(X), _ptr(Wt), _ptr(Y), M, N, K, variant, splits, _stream(stream)))


def w4a16_sparse24_repack(q, s, vp, idx, sp, K, N, group, stream=None):
    _check("w4a16_sparse24_repack", _lib.w4a16_sparse24_repack(
        _ptr(q), _ptr(s), _ptr(vp), _ptr(idx), _ptr(sp), K, N, group, _stream(stream)))


def w4a16_sparse24_unpack(vp, idx, sp, q, s, K, N, group, stream=None):
    _check("w4a16_sparse24_unpack", _lib.w4a16_sparse24_unpack(
        _ptr(vp), _ptr(idx), _ptr(sp), _ptr(q), _ptr(s), K, N, group, _stream(stream)))


def w4a16_sparse24_gemm(X, vp, idx, sp, Y, M, N, K, group, stream=None):
    _check("w4a16_sparse24_gemm", _lib.w4a16_sparse24_gemm(
        _ptr(X), _ptr(vp), _ptr(idx), _ptr(sp), _ptr(Y), M, N, K, group, _stream(stream)))


def w4a16_sparse24_gemm_plan(X, vp, idx, sp, Y, M, N, K, group, variant=-1, splits=0,
                             stream=None):
    _check("w4a16_sparse24_gemm_plan", _lib.w4a16_sparse24_gemm_plan(
        _ptr(X), _ptr(vp), _ptr(idx), _ptr(sp), _ptr(Y), M, N, K, group, variant, splits,
        _stream(stream)))


def w4a16_gemm_bf16(X, wp, sp, zp, Y, M, N, K, group, stream=None):
    _check("w4a16_gemm_bf16", _lib.w4a16_gemm_bf16(_ptr(X), _ptr(wp), _ptr(sp), _ptr(zp),
                                                   _ptr(Y), M, N, K, group, _stream(stream)))


def w4a16_gemm_bf16_plan(X, wp, sp, zp, Y, M, N, K, group, variant=-1, splits=0, stream=None):
    _check("w4a16_gemm_bf16_plan", _lib.w4a16_gemm_bf16_plan(
        _ptr(X), _ptr(wp), _ptr(sp), _ptr(zp), _ptr(Y), M, N, K, group, variant, splits,
        _stream(stream)))


def w4a16_gemm_bf16_variants() -> int:
    return _lib.w4a16_gemm_bf16_variants()


def w4a16_gemm_bf16_variant_name(v: int):
    r = _lib.w4a16_gemm_bf16_variant_name(v)
    return None if r is None else r.decode()


WS_COUNTER_BYTES = 65536  # W4A16_WS_COUNTER_BYTES


def w4a16_set_workspace(ptr, nbytes, stream=None):
    """Caller-owned workspace for launches on `stream` (ptr None: library-owned again)."""
    _check("w4a16_set_workspace", _lib.w4a16_set_workspace(_ptr(ptr), nbytes, _stream(stream)))


# ---- fp8 (E4M3) activations: W4A8 ---------------------------------------------------
def w4a8_gemm(X8, xscale, wp, sp, zp, Y, M, N, K, group, stream=None):
    _check("w4a8_gemm", _lib.w4a8_gemm(_ptr(X8), _ptr(xscale), _ptr(wp), _ptr(sp), _ptr(zp),
                                       _ptr(Y), M, N, K, group, _stream(stream)))


def w4a8_gemm_plan(X8, xscale, wp, sp, zp, Y, M, N, K, group, variant=-1, splits=0,
                   stream=None):
    _check("w4a8_gemm_plan", _lib.w4a8_gemm_plan(
        _ptr(X8), _ptr(xscale), _ptr(wp), _ptr(sp), _ptr(zp), _ptr(Y), M, N, K, group, variant,
        splits, _stream(stream)))


# ---- MXFP4 weights x fp8 activations (block scales inside the matrix instruction) --
def w4a8_mx_repack(q, e, wp, sp, K, N, stream=None):
    _check("w4a8_mx_repack", _lib.w4a8_mx_repack(_ptr(q), _ptr(e), _ptr(wp), _ptr(sp), K, N,
                                                 _stream(stream)))


def w4a8_mx_gemm(X8, xscale, wp, sp, Y, M, N, K, stream=None):
    _check("w4a8_mx_gemm", _lib.w4a8_mx_gemm(_ptr(X8), _ptr(xscale), _ptr(wp), _ptr(sp),
                                             _ptr(Y), M, N, K, _stream(stream)))


def w4a8_mx_gemm_plan(X8, xscale, wp, sp, Y, M, N, K, variant=-1, grid=0, stream=None):
    _check("w4a8_mx_gemm_plan", _lib.w4a8_mx_gemm_plan(
        _ptr(X8), _ptr(xscale), _ptr(wp), _ptr(sp), _ptr(Y), M, N, K, variant, grid,
        _stream(stream)))


def w4a8_mx_variants() -> int:
    return _lib.w4a8_mx_variants()


def w4a8_mx_variant_name(variant: int):
    n = _lib.w4a8_mx_variant_name(variant)
    return None if n is None else n.decode()


def alloc_mx(K: int, N: int, device="cuda"):
    """Empty device buffers (torch uint8) for the MXFP4 codes wp (K*N/2 bytes) and block
    scales sp (K*N/32 bytes) of w4a8_mx_repack."""
    import torch
    return (torch.empty(K * N // 2, dtype=torch.uint8, device=device),
            torch.empty(K * N // 32, dtype=torch.uint8, device=device))


# ---- calibration kernels ---------------------------------------------------------
def w4a16_probe_read(p, nbytes, out, stream=None):
    # the C entry point cannot see the buffer's size: refuse a read past a tensor's end
    if hasattr(p, "numel") and nbytes > p.numel() * p.element_size():
        raise ValueError(f"w4a16_probe_read: {nbytes} bytes past a {p.numel() * p.element_size()}"
                         "-byte tensor")
    _check("w4a16_probe_read", _lib.w4a16_probe_read(_ptr(p), nbytes, _ptr(out), _stream(stream)))


def w4a16_probe_mfma(workgroups, iters, out, stream=None):
    _check("w4a16_probe_mfma", _lib.w4a16_probe_mfma(workgroups, iters, _ptr(out), _stream(stream)))


def w4a16_probe_mfma_flops(workgroups: int, iters: int) -> float:
    return _lib.w4a16_probe_mfma_flops(workgroups, iters)


# ---- allocation helper (device memory through torch) ---------------------------
def alloc_packed(K: int, N: int, group: int, asym: bool, device="cuda"):
    """Empty device buffers (torch uint8) for the repacked wp, sp and zp."""
    import torch
    wp = torch.empty(w4a16_packed_bytes(K, N, group, BUF_W), dtype=torch.uint8, device=device)
    sp = torch.empty(w4a16_packed_bytes(K, N, group, BUF_S), dtype=torch.uint8, device=device)
    zp = (torch.empty(w4a16_packed_bytes(K, N, group, BUF_Z), dtype=torch.uint8, device=device)
          if asym else None)
    return wp, sp, zp


def alloc_sparse24(K: int, N: int, group: int, device="cuda"):
    """Empty device buffers (torch uint8) for the compressed vp, idx and sp."""
    import torch
    mk = lambda which: torch.empty(w4a16_packed_bytes(K, N, group, which), dtype=torch.uint8,
                                   device=device)
    return mk(BUF_SPARSE_V), mk(BUF_SPARSE_I), mk(BUF_SPARSE_S)
