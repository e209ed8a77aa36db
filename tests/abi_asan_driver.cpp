// Host-only driver for the sanitizer build of the C ABI (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library): exercises every query and
// the argument validation of every entry point with arguments that are refused on the host
// before any device call.
// Prints "ok" and returns 0 when every call returned what the interface promises.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "w4a16.h"

static int failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      std::printf("FAIL line %d: %s\n", __LINE__, #cond);        \
      ++failures;                                                 \
    }                                                             \
  } while (0)

int main(int argc, char** argv) {
  if (argc > 1 && std::strcmp(argv[1], "--planted-overflow") == 0) {
    // a heap overflow in the driver itself: the sanitizer must stop the program here
    volatile char* p = new char[16];
    p[16 + (argc > 5)] = 1;
    delete[] p;
    std::printf("planted overflow not caught\n");
    return 0;
  }
  EXPECT(w4a16_layout_version() == 1);
  for (int c = -12; c <= 2; ++c) EXPECT(w4a16_strerror(c) != nullptr && std::strlen(w4a16_strerror(c)) > 0);
  EXPECT(w4a16_strerror(42) != nullptr);

  // sizes: valid, invalid, and the largest accepted shapes
  const int Ks[] = {0, 64, 128, 256, 1024, 1 << 20, 1 << 25, 1 << 30, -128};
  const int Ns[] = {0, 8, 16, 48, 4096, 1 << 20, 1 << 26, -16};
  const int Gs[] = {0, 32, 64, 128, 192, 256, 1 << 20};
  for (int K : Ks)
    for (int N : Ns)
      for (int g : Gs)
        for (int which = -1; which <= 6; ++which) (void)w4a16_packed_bytes(K, N, g, which);
  EXPECT(w4a16_packed_bytes(4096, 4096, 128, 0) == (size_t)4096 * 4096 / 2);
  EXPECT(w4a16_packed_bytes(4096, 4096, 128, 9) == 0);

  // plans and workspace queries over many shapes (all host code)
  int out[4];
  const int Ms[] = {-1, 0, 1, 2, 4, 5, 8, 15, 16, 17, 32, 33, 48, 64, 65, 100, 128, 192, 255,
                    256, 300, 1024, 4096, 1 << 16, 1 << 20};
  const int KN[][2] = {{1024, 1024}, {4096, 4096}, {3072, 768},  {8192, 28672}, {28672, 8192},
                       {8192, 10240}, {128, 16},   {1 << 25, 16}, {1 << 23, 16}, {4096, 256},
                       {11008, 4096}, {4096, 11008}, {2560, 2560}, {100, 16}, {4096, 4100}};
  for (auto& kn : KN)
    for (int M : Ms) {
      for (int g : {64, 128, 256}) (void)w4a16_gemm_describe(M, kn[1], kn[0], g, out);
      (void)w4a16_workspace_bytes(M, kn[1], kn[0]);
    }
  EXPECT(w4a16_gemm_describe(1, 4096, 4096, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_gemm_describe(0, 4096, 4096, 128, out) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm_describe(128, 16, 1 << 25, 128, out) == W4A16_ERR_SHAPE);
  for (int v = -2; v <= w4a16_gemm_variants() + 1; ++v) (void)w4a16_gemm_variant_name(v);
  for (int v = -2; v <= w4a16_fp16_gemm_variants() + 1; ++v) (void)w4a16_fp16_gemm_variant_name(v);
  for (int v = -2; v <= w4a8_mx_variants() + 1; ++v) (void)w4a8_mx_variant_name(v);
  for (int v = -2; v <= w4a16_gemm_bf16_variants() + 1; ++v) (void)w4a16_gemm_bf16_variant_name(v);
  EXPECT(w4a16_gemm_bf16_variant_name(w4a16_gemm_bf16_variants()) == nullptr);
  EXPECT(w4a16_gemm_variant_name(-1) == nullptr);

  // argument validation: refused on the host, nothing enqueued
  alignas(16) static unsigned char buf[256];
  void* A = buf;           // aligned, never dereferenced by a refused call
  void* MIS = buf + 2;     // misaligned
  const uint16_t* X = static_cast<const uint16_t*>(A);
  uint16_t* Y = static_cast<uint16_t*>(A);
  EXPECT(w4a16_gemm(nullptr, A, X, nullptr, Y, 16, 1024, 1024, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_gemm(X, A, X, nullptr, Y, 16, 1000, 1024, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm(X, A, X, nullptr, Y, 16, 1024, 1000, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm(X, A, X, nullptr, Y, 0, 1024, 1024, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm(X, A, X, nullptr, Y, 16, 1024, 1024, 96, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm(static_cast<const uint16_t*>(MIS), A, X, nullptr, Y, 16, 1024, 1024, 128,
                    nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_gemm(X, A, X, nullptr, Y, 128, 16, 1 << 25, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm_noalloc(X, A, X, nullptr, Y, 16, 1000, 1024, 128, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm_plan(X, A, X, nullptr, Y, 16, 1024, 1024, 128, -2, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_plan(X, A, X, nullptr, Y, 16, 1024, 1024, 128, 0, -1, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_gemm_plan(X, A, X, nullptr, Y, 16, 1024, 1024, 128, w4a16_gemm_variants(), 0,
                         nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_repack(nullptr, X, nullptr, A, Y, nullptr, 1024, 1024, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_repack(static_cast<const int32_t*>(A), X, static_cast<const int32_t*>(A), A, Y,
                      nullptr, 1024, 1024, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_unpack(A, X, nullptr, static_cast<int32_t*>(A), Y, nullptr, 1024, 1000, 128,
                      nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_dequant(static_cast<const int32_t*>(A), X, nullptr, Y, 1024, 1024, 100,
                       nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_fp16_gemm(X, X, Y, 16, 1024, 1000, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_fp16_gemm(X, X, Y, 1, 16, 1 << 26, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_fp16_gemm_plan(X, X, Y, 16, 1024, 1024, -3, 0, nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_sparse24_gemm(X, A, nullptr, X, Y, 16, 1024, 1024, 128, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_sparse24_gemm(X, A, A, X, Y, 16, 1024, 1024, 64, nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_sparse24_repack(static_cast<const int32_t*>(A), X, A, A, Y, 1024, 1024, 64,
                               nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_gemm_bf16_plan(X, A, X, nullptr, Y, 16, 1024, 1024, 128,
                              w4a16_gemm_bf16_variants(), 0, nullptr) == W4A16_ERR_ARG);
  const uint8_t* X8 = static_cast<const uint8_t*>(A);
  EXPECT(w4a8_gemm(X8, reinterpret_cast<const float*>(buf + 2), A, X, nullptr, Y, 16, 1024, 1024,
                   128, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a8_gemm_plan(X8, nullptr, A, X, nullptr, Y, 16, 1024, 1024, 128, -5, 0, nullptr) ==
         W4A16_ERR_ARG);
  EXPECT(w4a8_mx_gemm_plan(X8, nullptr, A, A, Y, 16, 1024, 1024, w4a8_mx_variants(), 0,
                           nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a8_mx_repack(nullptr, X8, A, A, 1024, 1024, nullptr) == W4A16_ERR_NULL);
  EXPECT(w4a16_set_workspace(MIS, 1 << 20, nullptr) == W4A16_ERR_ALIGN);
  EXPECT(w4a16_probe_read(A, 15, static_cast<uint32_t*>(A), nullptr) == W4A16_ERR_SHAPE);
  EXPECT(w4a16_probe_mfma(0, 1, static_cast<float*>(A), nullptr) == W4A16_ERR_ARG);
  EXPECT(w4a16_probe_mfma_flops(0, 1) == 0.0);
  // (no call here passes validation: the pointers above are host memory)
  if (failures) return 1;
  std::printf("ok\n");
  return 0;
}
