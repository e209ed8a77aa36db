// MXFP4 weights x fp8 activations for decode-sized batches (M <= 32) on gfx950.
//
// The format and the instruction are those of the tiled kernel's MXFP4 mode (FP4 codes
// with E8M0 micro-block scales that the matrix unit applies itself, dingiv.github.io
// "Marlin", section "与 Blackwell NVFP4 的对比"); at small M the product is bound by
// streaming the weights once, so this kernel keeps the path short:
//   * a workgroup of 4 waves owns NT column tiles of 16 columns; wave w takes the
//     128-row k-blocks w, w + 4, ... (neighbouring 1 KiB blocks are read together);
//   * each lane loads its 16 code bytes and its scale byte of a block straight into
//     registers (non-temporal: every weight byte is used once), and its X fragment of each
//     of the MR 16-row tiles (the FP8 operand's K order: chunks g and 4+g of row
//     16i + l%16 of the k-block, g = l/16) from L2, zeros for rows past M;
//   * v_mfma_scale_f32_16x16x128_f8f6f4 with the codes as the FP4 operand and their
//     scale byte, X as the FP8 operand with unit scale;
//   * the 4 waves' sums are added in LDS in wave order (bitwise reproducible), the fp32
//     row scale applied, and Y rounded once to fp16.
// Many small workgroups (one per NT column tiles) keep enough loads in flight; there is
// no barrier inside the k loop.
#include "internal.h"

namespace w4a16 {

namespace {

typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int int8v __attribute__((ext_vector_type(8)));

constexpr int DW = 4;  // waves per workgroup

template <int NT, int MR>
__global__ __launch_bounds__(64 * DW) void mx_decode_kernel(
    const uint8_t* __restrict__ X, const float* __restrict__ xscale,
    const u32x4* __restrict__ W, const uint8_t* __restrict__ S, uint16_t* __restrict__ Y, int M,
    int N, int K) {
  __shared__ float4v red[DW][MR * NT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int Gk = K / KBLK;
  const int ntiles = N / 16;
  const int t0 = blockIdx.x * NT;
  const int r = lane & 15, g = lane >> 4;
  bool row_ok[MR];
  const uint8_t* xr[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    row_ok[i] = r + 16 * i < M;
    xr[i] = X + (size_t)(row_ok[i] ? r + 16 * i : 0) * K + 16 * g;
  }

  float4v acc[MR][NT];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = float4v{0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](int kb, int i) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (row_ok[i]) {
      lo = *reinterpret_cast<const u32x4*>(xr[i] + (size_t)kb * KBLK);
      hi = *reinterpret_cast<const u32x4*>(xr[i] + (size_t)kb * KBLK + 64);
    }
    return int8v{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  // two k-blocks per trip: the second block's loads are in flight while the first
  // block's matrix instructions wait for theirs
  int kb = wave;
  for (; kb + DW < Gk; kb += 2 * DW) {
    u32x4 w0[NT], w1[NT];
    int s0[NT], s1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tt = t0 + t < ntiles ? t0 + t : ntiles - 1;  // past N: recompute the last tile
      const size_t b0 = ((size_t)tt * Gk + kb) * 64 + lane;
      const size_t b1 = b0 + (size_t)DW * 64;
      w0[t] = __builtin_nontemporal_load(W + b0);
      w1[t] = __builtin_nontemporal_load(W + b1);
      s0[t] = (int)__builtin_nontemporal_load(S + b0);
      s1[t] = (int)__builtin_nontemporal_load(S + b1);
    }
    int8v x0[MR], x1[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      x0[i] = load_x(kb, i);
      x1[i] = load_x(kb + DW, i);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int8v b = {(int)w0[t][0], (int)w0[t][1], (int)w0[t][2], (int)w0[t][3], 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < MR; ++i)
        acc[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, x0[i], acc[i][t], 4, 0, 0,
                                                                     s0[t], 0, 127);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int8v b = {(int)w1[t][0], (int)w1[t][1], (int)w1[t][2], (int)w1[t][3], 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < MR; ++i)
        acc[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, x1[i], acc[i][t], 4, 0, 0,
                                                                     s1[t], 0, 127);
    }
  }
  if (kb < Gk) {  // a last single k-block
    int8v x0[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) x0[i] = load_x(kb, i);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tt = t0 + t < ntiles ? t0 + t : ntiles - 1;
      const size_t b0 = ((size_t)tt * Gk + kb) * 64 + lane;
      const u32x4 w = __builtin_nontemporal_load(W + b0);
      const int s = (int)__builtin_nontemporal_load(S + b0);
      const int8v b = {(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < MR; ++i)
        acc[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b, x0[i], acc[i][t], 4, 0, 0,
                                                                     s, 0, 127);
    }
  }

#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][i * NT + t][lane] = acc[i][t];
  __syncthreads();
  // wave w finishes the (row tile, column tile) pairs w, w + 4, ...: lane l holds row
  // 16i + l%16 and columns 4(l/16) .. +3 of the tile
  for (int p = wave; p < MR * NT; p += DW) {
    const int i = p / NT, t = p - i * NT;
    if (t0 + t >= ntiles) continue;
    float4v v = red[0][p][lane];
#pragma unroll
    for (int w = 1; w < DW; ++w) v += red[w][p][lane];
    const int row = r + 16 * i;
    if (row < M) {
      const float xs = xscale != nullptr ? xscale[row] : 1.0f;
      v *= xs;
      const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
      const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2*>(Y + (size_t)row * N + (size_t)(t0 + t) * 16 + 4 * g) =
          u32x2{lo, hi};
    }
  }
}

typedef void (*MxDecodeFn)(const uint8_t*, const float*, const u32x4*, const uint8_t*, uint16_t*,
                           int, int, int);
// fn1: one 16-row tile (M <= 16), fn2: two (M <= 32)
struct MxDecodeVariant {
  int NT;
  MxDecodeFn fn1, fn2;
  const char* name;
};
const MxDecodeVariant kMxDecode[] = {
    {1, mx_decode_kernel<1, 1>, mx_decode_kernel<1, 2>, "mx_decode_nt1"},
    {2, mx_decode_kernel<2, 1>, mx_decode_kernel<2, 2>, "mx_decode_nt2"},
    {4, mx_decode_kernel<4, 1>, mx_decode_kernel<4, 2>, "mx_decode_nt4"},
};
constexpr int kNumMxDecode = sizeof(kMxDecode) / sizeof(kMxDecode[0]);

}  // namespace

int mx_decode_variant_count() { return kNumMxDecode; }
const char* mx_decode_variant_name(int v) {
  return v >= 0 && v < kNumMxDecode ? kMxDecode[v].name : nullptr;
}

hipError_t mx_decode_launch(int variant, const uint8_t* X, const float* xscale, const void* wp,
                            const uint8_t* sp, uint16_t* Y, int M, int N, int K, hipStream_t st) {
  if (variant < 0 || variant >= kNumMxDecode || M < 1 || M > 32) return hipErrorInvalidValue;
  const MxDecodeVariant& v = kMxDecode[variant];
  const int ntiles = N / 16;
  const int wgs = (ntiles + v.NT - 1) / v.NT;
  hipLaunchKernelGGL(M > 16 ? v.fn2 : v.fn1, dim3(wgs), dim3(64 * DW), 0, st, X, xscale,
                     reinterpret_cast<const u32x4*>(wp), sp, Y, M, N, K);
  return hipGetLastError();
}

}  // namespace w4a16
