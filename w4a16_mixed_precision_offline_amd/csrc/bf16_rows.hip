// bf16 and fp8 activations rewritten as fp16 rows for the fp16 tiled kernel.
//
// The pages run the fused product on 16-bit activations ("Marlin / GPTQ-Marlin",
// brain.gartu.xyz, section "1. Le problème": W4A16 means fp16/bf16 activations).  With bf16
// activations the weights cannot become fp16-exact dequantized values inside a bf16 matrix
// instruction (bf16 keeps 8 significant bits), so for larger batches each row of X is
// rewritten in fp16, which keeps 11: the row is multiplied by a power of two 2^d chosen
// from its largest finite magnitude, and the inverse power 2^-d is kept per row and applied
// by the GEMM to the finished fp32 sums (an exact scaling).
//
// Exactness.  d puts the row's largest finite |x| in [2^15, 2^16); a bf16 value there is at
// most (2 - 2^-7) * 2^15 = 65280, below the fp16 maximum 65504.  A bf16 value whose scaled
// exponent is -17 or more has a unit in the last place of 2^-24 or coarser, which fp16
// holds exactly (its subnormal step is 2^-24); so every value within 2^32 of the row's
// maximum is carried exactly, and smaller ones round to the fp16 subnormal grid (an error
// of at most 2^-40 of the row's maximum).  d is kept in [-126, 126] so both powers are
// normal fp32 numbers; only a row whose maximum lies below 2^-111 is then scaled less.
// Infinities and NaNs are left out of the maximum and stay infinities and NaNs.
//
// FP8 activations (the W4A8 variant, dingiv.github.io "Marlin", section "CUTLASS W4A8
// （混合精度）") take the same route above 32 rows: every E4M3 code is an fp16 value, so
// their rows are converted as they are and the caller's fp32 row scale goes to the sums.
#include "internal.h"

namespace w4a16 {

namespace {

constexpr int kRowThreads = 256;
constexpr int kHeld = 16;  // 16-byte chunks a thread keeps in registers: K <= 32768

// largest finite bf16 magnitude (bits without the sign; 0x7F80 and above are inf / NaN)
__device__ __forceinline__ uint32_t finite_mag(uint32_t h) {
  const uint32_t m = h & 0x7FFFu;
  return m < 0x7F80u ? m : 0u;
}
__device__ __forceinline__ uint32_t chunk_max(const uint4& v) {
  uint32_t m = 0;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = max(m, finite_mag(w[i] & 0xFFFFu));
    m = max(m, finite_mag(w[i] >> 16));
  }
  return m;
}

// Power d of the row scale from the largest finite magnitude (bf16 bits without sign).
__device__ __forceinline__ int row_shift(uint32_t mag) {
  if (mag == 0) return 0;
  const int e = (int)(mag >> 7);
  // normal: |x| in [2^(e-127), 2^(e-126)); subnormal: |x| = f * 2^-133 with f = mag
  const int top = e > 0 ? e - 127 : (31 - __clz((int)mag)) - 133;
  int d = 15 - top;
  d = d < -126 ? -126 : d;
  d = d > 126 ? 126 : d;
  return d;
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t w, float up) {
  const float lo = __uint_as_float(w << 16) * up;
  const float hi = __uint_as_float(w & 0xFFFF0000u) * up;
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;  // nearest-even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}
__device__ __forceinline__ uint4 scale_chunk(const uint4& v, float up) {
  return uint4{scale_pair(v.x, up), scale_pair(v.y, up), scale_pair(v.z, up),
               scale_pair(v.w, up)};
}

// One workgroup per row of X.  HOLD: the row fits in registers (K <= 8 * 256 * kHeld) and
// is read once; otherwise it is read twice (the second read mostly from L2).
template <bool HOLD>
__global__ __launch_bounds__(kRowThreads) void bf16_rows_kernel(const uint16_t* __restrict__ X,
                                                                uint16_t* __restrict__ Xh,
                                                                float* __restrict__ rscale,
                                                                int K) {
  const size_t row = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(X + row * (size_t)K);
  uint4* dst = reinterpret_cast<uint4*>(Xh + row * (size_t)K);
  const int chunks = K / 8;
  const int tid = threadIdx.x;
  uint32_t mx = 0;
  uint4 held[HOLD ? kHeld : 1];
  if constexpr (HOLD) {
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
      const int c = tid + j * kRowThreads;
      held[j] = c < chunks ? src[c] : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kHeld; ++j) mx = max(mx, chunk_max(held[j]));
  } else {
    for (int c = tid; c < chunks; c += kRowThreads) mx = max(mx, chunk_max(src[c]));
  }
  // workgroup maximum: across the wave, then across the four waves through LDS
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  __shared__ uint32_t wmax[kRowThreads / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = mx;
  __syncthreads();
  mx = 0;
#pragma unroll
  for (int w = 0; w < kRowThreads / 64; ++w) mx = max(mx, wmax[w]);
  const int d = row_shift(mx);
  const float up = __builtin_ldexpf(1.0f, d);
  if (tid == 0) rscale[row] = __builtin_ldexpf(1.0f, -d);
  if constexpr (HOLD) {
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
      const int c = tid + j * kRowThreads;
      if (c < chunks) dst[c] = scale_chunk(held[j], up);
    }
  } else {
    for (int c = tid; c < chunks; c += kRowThreads) dst[c] = scale_chunk(src[c], up);
  }
}

// OCP FP8 E4M3 (sign, 4 exponent bits of bias 7, 3 mantissa bits, no infinities, S.1111.111
// NaN) to fp16 bits.  Every E4M3 value is an fp16 value: normal codes (1 + m/8) * 2^(e-7)
// with e = 1..15 land on fp16 exponents -6..8, subnormal codes m * 2^-9 on fp16 normals, so
// the conversion is exact and the row needs no scale of its own (the caller's row scale,
// if any, is applied to the finished sums).
__device__ __forceinline__ uint32_t e4m3_to_f16_bits(uint32_t b) {
  const uint32_t sign = (b & 0x80u) << 8;
  const uint32_t em = b & 0x7Fu;
  if (em == 0x7Fu) return sign | 0x7E00u;
  const int e = (int)(em >> 3);
  const uint32_t m = em & 7u;
  const float v = e > 0 ? __builtin_ldexpf((float)(8u | m), e - 10)
                        : __builtin_ldexpf((float)m, -9);
  return sign | (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}
__device__ __forceinline__ uint32_t e4m3_pair(uint32_t w, int sh) {
  return e4m3_to_f16_bits((w >> sh) & 0xFFu) | (e4m3_to_f16_bits((w >> (sh + 8)) & 0xFFu) << 16);
}

// 16 codes per thread per step (one 16-byte load, two 16-byte stores), grid-stride.
__global__ __launch_bounds__(256) void fp8_rows_kernel(const uint4* __restrict__ X8,
                                                       uint4* __restrict__ Xh, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * blockDim.x) {
    const uint4 v = X8[i];
    Xh[2 * i] = uint4{e4m3_pair(v.x, 0), e4m3_pair(v.x, 16), e4m3_pair(v.y, 0), e4m3_pair(v.y, 16)};
    Xh[2 * i + 1] =
        uint4{e4m3_pair(v.z, 0), e4m3_pair(v.z, 16), e4m3_pair(v.w, 0), e4m3_pair(v.w, 16)};
  }
}

}  // namespace

hipError_t launch_fp8_rows_to_f16(const uint8_t* X8, uint16_t* Xh, size_t elems, hipStream_t st) {
  if (elems == 0 || elems % 16 != 0) return hipErrorInvalidValue;
  const size_t n16 = elems / 16;
  const size_t want = (n16 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 8192 ? want : 8192);
  hipLaunchKernelGGL(fp8_rows_kernel, dim3(blocks), dim3(256), 0, st,
                     reinterpret_cast<const uint4*>(X8), reinterpret_cast<uint4*>(Xh), n16);
  return hipGetLastError();
}

hipError_t launch_bf16_rows_to_f16(const uint16_t* X, uint16_t* Xh, float* rscale, int M, int K,
                                   hipStream_t st) {
  if (M <= 0 || K <= 0 || K % 8 != 0) return hipErrorInvalidValue;
  if (K <= 8 * kRowThreads * kHeld)
    hipLaunchKernelGGL(bf16_rows_kernel<true>, dim3(M), dim3(kRowThreads), 0, st, X, Xh, rscale,
                       K);
  else
    hipLaunchKernelGGL(bf16_rows_kernel<false>, dim3(M), dim3(kRowThreads), 0, st, X, Xh,
                       rscale, K);
  return hipGetLastError();
}

}  // namespace w4a16
