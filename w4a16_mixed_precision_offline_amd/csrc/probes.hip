// Calibration kernels: the achievable ceilings on this GPU that the GEMM's measured
// rates are set against, next to the published peaks.
//   * probe_read_kernel: a plain streaming read of a buffer (16-byte non-temporal
//     loads, every byte once), i.e. the best a kernel that only has to read the same
//     weight bytes could do at that size, launch and ramp included.
//   * probe_mfma_kernel: independent chains of dense fp16 matrix instructions with no
//     memory traffic, i.e. the matrix rate at the clock the chip holds under sustained
//     matrix load.
// Their results feed nothing: each kernel writes its output word only when a data-
// dependent value equals a sentinel, so the compiler cannot drop the work.
#include "internal.h"

namespace w4a16 {

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;
constexpr uint32_t kSentinel = 0x9E3779B9u;

// n16 16-byte words; each thread XORs the words i, i + stride, ... (stride = all
// threads of the grid), four loads in flight per iteration.
__global__ __launch_bounds__(kReadThreads) void probe_read_kernel(const u32x4* __restrict__ p,
                                                                  size_t n16,
                                                                  uint32_t* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // the XOR over the whole buffer of the lanes' partial values is not formed: a single
  // lane seeing the sentinel is enough to keep the loads (and lets a test place it)
  if (acc == kSentinel) out[0] = acc;
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_f16 per wave: measured on
// MI355X to reach 97% of the 2.5166 PFLOP/s nominal peak with one wave per SIMD, while
// v_mfma_f32_16x16x32_f16 needs 16 independent chains per wave for 90% (its result
// latency is several times its issue interval), so the larger shape is the ceiling.
constexpr int kMfmaChains = 4;
typedef float float16v __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  half8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (_Float16)(float)((lane + e) & 7);
    b[e] = (_Float16)(float)((lane * 3 + e) & 7);
  }
  float16v c[kMfmaChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j)
      c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += c[j][r];
  if (s == -1.0f) out[0] = s;  // never: every product is non-negative
}

}  // namespace

hipError_t launch_probe_read(const void* p, size_t bytes, uint32_t* out, hipStream_t st) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + (size_t)kReadThreads * kReadUnroll - 1) / ((size_t)kReadThreads * kReadUnroll);
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, st,
                     static_cast<const u32x4*>(p), n16, out);
  return hipGetLastError();
}

hipError_t launch_probe_mfma(int workgroups, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(256), 0, st, iters, out);
  return hipGetLastError();
}

double probe_mfma_flops(int workgroups, int iters) {
  // 4 waves per workgroup, kMfmaChains instructions per iteration, 32x32x16 each
  return (double)workgroups * 4 * iters * kMfmaChains * (2.0 * 32 * 32 * 16);
}

}  // namespace w4a16
