"""Drop-in linear layer over the W4A16 GEMM: a torch module that holds a weight in the
repacked 4-bit layout (repacked once, when the layer is built) and whose forward is one
call of w4a16_gemm.  The pages describe the same split: weights and scales are
reshuffled once at load time ("Marlin / GPTQ-Marlin", brain.gartu.xyz, section "2. Tiled
layout et repacking") and the layer then calls the kernel directly ("Marlin Project
Overview", vecbase.com, usage section: a layer that converts the quantized weights and
calls the kernel).

The module does no arithmetic of its own: it validates shapes, reshapes the input to a
row-major [M, K] matrix and forwards to the library, which fails loudly if it is not
built.  Quantizing a float weight (GPTQ, AWQ, ...) is outside this library: the module
takes already quantized codes, scales and optional zero-points in the canonical format
of w4a16_repack.
"""
from __future__ import annotations

import torch

from . import (alloc_mx, alloc_packed, w4a8_gemm, w4a8_mx_gemm, w4a8_mx_repack, w4a16_gemm,
               w4a16_gemm_bf16, w4a16_packed_bytes, w4a16_repack, w4a16_unpack, BUF_W)


class W4A16Linear(torch.nn.Module):
    """y = x @ W for x [..., in_features] and a group-quantized 4-bit W [in_features,
    out_features] (w = (q - z) * s, z = 8 without zero-points).

    x may be fp16 (y fp16, w4a16_gemm), bf16 (y bf16, w4a16_gemm_bf16) or already
    quantized FP8 E4M3 (torch.float8_e4m3fn) with an optional fp32 scale per row
    `xscale` of shape x.shape[:-1] (y fp16, w4a8_gemm: INT4 weights times FP8
    activations, "Marlin", dingiv.github.io, section "CUTLASS W4A8（混合精度）")."""

    def __init__(self, in_features: int, out_features: int, group: int = 128,
                 zero_points: bool = False, device="cuda"):
        super().__init__()
        if w4a16_packed_bytes(in_features, out_features, group, BUF_W) == 0:
            raise ValueError(
                f"unsupported shape: in_features={in_features} (multiple of 128 and of the "
                f"group), out_features={out_features} (multiple of 16), group={group} "
                "(64 or a multiple of 128)")
        self.in_features = in_features
        self.out_features = out_features
        self.group = group
        wp, sp, zp = alloc_packed(in_features, out_features, group, zero_points, device=device)
        self.register_buffer("wp", wp)
        self.register_buffer("sp", sp)
        self.register_buffer("zp", zp)

    @classmethod
    def from_quantized(cls, q: torch.Tensor, s: torch.Tensor, z: torch.Tensor | None = None,
                       group: int = 128) -> "W4A16Linear":
        """Build from canonical device tensors: q int32 [K/8, N] (8 codes per word along K),
        s fp16 [K/group, N], z int32 [K/group, N/8] or None; repacks them once."""
        if q.dtype != torch.int32 or s.dtype != torch.float16 or (z is not None and z.dtype != torch.int32):
            raise TypeError("q and z must be int32, s float16")
        K, N = q.shape[0] * 8, q.shape[1]
        if tuple(s.shape) != (K // group, N) or (z is not None and tuple(z.shape) != (K // group, N // 8)):
            raise ValueError("s must be [K/group, N] and z [K/group, N/8]")
        layer = cls(K, N, group, z is not None, device=q.device)
        w4a16_repack(q.contiguous(), s.contiguous(), None if z is None else z.contiguous(),
                     layer.wp, layer.sp, layer.zp, K, N, group)
        return layer

    def unpack(self):
        """The canonical (q, s, z) this layer holds (z None without zero-points)."""
        K, N, g = self.in_features, self.out_features, self.group
        q = torch.empty((K // 8, N), dtype=torch.int32, device=self.wp.device)
        s = torch.empty((K // g, N), dtype=torch.float16, device=self.wp.device)
        z = (torch.empty((K // g, N // 8), dtype=torch.int32, device=self.wp.device)
             if self.zp is not None else None)
        w4a16_unpack(self.wp, self.sp, self.zp, q, s, z, K, N, g)
        return q, s, z

    def forward(self, x: torch.Tensor, xscale: torch.Tensor | None = None) -> torch.Tensor:
        fp8 = x.dtype == torch.float8_e4m3fn
        if x.dtype not in (torch.float16, torch.bfloat16) and not fp8:
            raise TypeError(f"expected float16, bfloat16 or float8_e4m3fn activations, got {x.dtype}")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"last dimension {x.shape[-1]} != in_features {self.in_features}")
        lead = x.shape[:-1]
        if xscale is not None:
            if not fp8:
                raise ValueError("xscale applies to float8_e4m3fn activations only")
            if xscale.dtype != torch.float32 or tuple(xscale.shape) != tuple(lead):
                raise ValueError(f"xscale must be float32 of shape {tuple(lead)}")
        x2 = x.reshape(-1, self.in_features).contiguous()
        M = x2.shape[0]
        y = torch.empty((M, self.out_features),
                        dtype=torch.bfloat16 if x.dtype == torch.bfloat16 else torch.float16,
                        device=x.device)
        if M > 0:
            args = (self.wp, self.sp, self.zp, y, M, self.out_features, self.in_features,
                    self.group)
            if fp8:
                a = None if xscale is None else xscale.reshape(-1).contiguous()
                w4a8_gemm(x2, a, *args)
            elif x.dtype == torch.bfloat16:
                w4a16_gemm_bf16(x2, *args)
            else:
                w4a16_gemm(x2, *args)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"group={self.group}, zero_points={self.zp is not None}")


class MXFP4Linear(torch.nn.Module):
    """y = x @ W for FP8 E4M3 activations x [..., in_features] (torch.float8_e4m3fn, with
    an optional fp32 scale per row `xscale` of shape x.shape[:-1]) and MXFP4 weights W
    [in_features, out_features]: w = e2m1(q) * 2^(e - 127), one E8M0 byte e per 32 rows of
    a column.  The block scales are applied by the matrix instruction itself (FP4 weights
    with micro-block scales, "Marlin", dingiv.github.io, section "与 Blackwell NVFP4 的对比");
    forward is one w4a8_mx_gemm call, y is fp16.  Weights are repacked once, when the
    layer is built."""

    def __init__(self, in_features: int, out_features: int, device="cuda"):
        super().__init__()
        if in_features <= 0 or in_features % 128 or out_features <= 0 or out_features % 16:
            raise ValueError(f"unsupported shape: in_features={in_features} (multiple of 128), "
                             f"out_features={out_features} (multiple of 16)")
        self.in_features = in_features
        self.out_features = out_features
        wp, sp = alloc_mx(in_features, out_features, device=device)
        self.register_buffer("wp", wp)
        self.register_buffer("sp", sp)

    @classmethod
    def from_quantized(cls, q: torch.Tensor, e: torch.Tensor) -> "MXFP4Linear":
        """Build from canonical device tensors: q int32 [K/8, N] (8 E2M1 codes per word along
        K, low nibble first), e uint8 [K/32, N] (E8M0 scale bytes); repacks them once."""
        if q.dtype != torch.int32 or e.dtype != torch.uint8:
            raise TypeError("q must be int32 and e uint8")
        K, N = q.shape[0] * 8, q.shape[1]
        if tuple(e.shape) != (K // 32, N):
            raise ValueError("e must be [K/32, N]")
        layer = cls(K, N, device=q.device)
        w4a8_mx_repack(q.contiguous(), e.contiguous(), layer.wp, layer.sp, K, N)
        return layer

    def forward(self, x: torch.Tensor, xscale: torch.Tensor | None = None) -> torch.Tensor:
        if x.dtype != torch.float8_e4m3fn:
            raise TypeError(f"expected float8_e4m3fn activations, got {x.dtype}")
        if x.shape[-1] != self.in_features:
            raise ValueError(f"last dimension {x.shape[-1]} != in_features {self.in_features}")
        lead = x.shape[:-1]
        if xscale is not None and (xscale.dtype != torch.float32 or tuple(xscale.shape) != tuple(lead)):
            raise ValueError(f"xscale must be float32 of shape {tuple(lead)}")
        x2 = x.reshape(-1, self.in_features).contiguous()
        M = x2.shape[0]
        y = torch.empty((M, self.out_features), dtype=torch.float16, device=x.device)
        if M > 0:
            a = None if xscale is None else xscale.reshape(-1).contiguous()
            w4a8_mx_gemm(x2, a, self.wp, self.sp, y, M, self.out_features, self.in_features)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return f"in_features={self.in_features}, out_features={self.out_features}, format=mxfp4"
