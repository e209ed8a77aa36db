// C ABI of libw4a16: argument validation (pure host code, runs before any HIP
// call), device check, per-(device, stream) split-K workspace, and dispatch to
// the kernels.  The interface and its rules are documented in include/w4a16.h.
#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/w4a16.h"
#include "internal.h"

using namespace w4a16;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape rules shared by the weight-format entry points.
int check_weight_shape(int K, int N, int group) {
  if (K <= 0 || N <= 0 || group <= 0) return W4A16_ERR_SHAPE;
  // groups of 64 rows, or whole multiples of the 128-row block
  if ((group != 64 && group % KBLK != 0) || K % KBLK != 0 || K % group != 0 || N % NTILE != 0)
    return W4A16_ERR_SHAPE;
  // word and block indices are 32-bit inside the kernels' per-dimension math
  if ((long long)K * N / 8 > (1LL << 31) - 1) return W4A16_ERR_SHAPE;
  return W4A16_OK;
}

// Device check: the current device must exist and be a gfx950.  Cached per device.
std::mutex g_mu;
std::map<int, int> g_dev_ok;  // device -> 1 ok / 0 not gfx950

int check_device(int* dev_out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return W4A16_ERR_DEVICE;
  }
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_dev_ok.find(dev);
  if (it == g_dev_ok.end()) {
    hipDeviceProp_t prop;
    int ok = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess)
      ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
    else
      (void)hipGetLastError();
    it = g_dev_ok.emplace(dev, ok).first;
  }
  if (dev_out) *dev_out = dev;
  return it->second ? W4A16_OK : W4A16_ERR_DEVICE;
}

// Split-K workspace: [counters (ints, zero at rest) | partials (floats)], one per
// (device, stream).  Counters are reset by the kernels themselves, so the buffer
// is cleared only when it is (re)allocated.
struct Workspace {
  void* ptr = nullptr;
  size_t counter_ints = 0;
  size_t part_floats = 0;
  bool external = false;  // caller-owned (w4a16_set_workspace): never grown or freed
};
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
// Library-owned buffers replaced by a larger one.  They are never freed: launches still in
// flight, and HIP graphs captured earlier, may hold their addresses.  Growth at least
// doubles the buffer, so what is kept here stays below the size of the live buffer.
std::vector<void*> g_retired;

// True when `st` is being captured into a graph (or its capture state is unknown): no
// allocation, clearing or synchronization may be issued then.
bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return cs != hipStreamCaptureStatusNone;
}

int get_workspace(int dev, hipStream_t st, size_t counters, size_t floats, int** cnt,
                  float** part) {
  *cnt = nullptr;
  *part = nullptr;
  if (counters == 0 && floats == 0) return W4A16_OK;
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_ws[std::make_pair(dev, st)];
  if (ws.external) {
    if (ws.counter_ints < counters || ws.part_floats < floats) return W4A16_ERR_WORKSPACE;
  } else if (ws.ptr == nullptr || ws.counter_ints < counters || ws.part_floats < floats) {
    // a graph being captured cannot take the allocation and the clearing of the counters:
    // the first call of a shape on a stream must come before any capture on it
    if (capturing(st)) return W4A16_ERR_WORKSPACE;
    size_t c = counters > ws.counter_ints ? counters : ws.counter_ints;
    size_t f = floats > ws.part_floats ? floats : ws.part_floats;
    if (ws.ptr) {
      if (c > ws.counter_ints && c < 2 * ws.counter_ints) c = 2 * ws.counter_ints;
      if (f > ws.part_floats && f < 2 * ws.part_floats) f = 2 * ws.part_floats;
    }
    c = (c + 63) / 64 * 64;  // keep the partials 256-byte aligned
    void* p = nullptr;
    if (hipMalloc(&p, c * sizeof(int) + f * sizeof(float)) != hipSuccess) {
      (void)hipGetLastError();
      return W4A16_ERR_WORKSPACE;
    }
    if (hipMemsetAsync(p, 0, c * sizeof(int), st) != hipSuccess) {
      (void)hipGetLastError();
      (void)hipFree(p);
      return W4A16_ERR_WORKSPACE;
    }
    if (ws.ptr) g_retired.push_back(ws.ptr);
    ws.ptr = p;
    ws.counter_ints = c;
    ws.part_floats = f;
  }
  *cnt = static_cast<int*>(ws.ptr);
  *part = reinterpret_cast<float*>(static_cast<int*>(ws.ptr) + ws.counter_ints);
  return W4A16_OK;
}

// ---- fixed device scratch for w4a16_gemm_noalloc ----------------------------------------
// [counters (W4A16_WS_COUNTER_BYTES, zero at rest) | fp32 partials].  128 MiB of partials
// hold the largest automatic plan: two 128 x 512 fp32 stream-K pieces per persistent
// workgroup of the eight-wave tiles, 256 workgroups.  In host code `scratch` only stands in for the symbol; the
// device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchPartBytes = (size_t)128 << 20;
constexpr size_t kScratchBytes = (size_t)W4A16_WS_COUNTER_BYTES + kScratchPartBytes;
static_assert(kScratchBytes == W4A16_NOALLOC_SCRATCH_BYTES, "header and library disagree");
std::map<int, char*> g_scratch;  // device -> device address of its copy of `scratch`

__global__ void clear_words_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

// The device address of this device's scratch array; on the first call for a device it
// is looked up and its counter region cleared by a small kernel on `st` (no memset node,
// so the clearing may also be captured into a graph and replayed).
int scratch_for_device(int dev, hipStream_t st, char** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it != g_scratch.end()) {
    *out = it->second;
    return W4A16_OK;
  }
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return W4A16_ERR_DEVICE;
  }
  const int words = W4A16_WS_COUNTER_BYTES / 4;
  hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, st,
                     static_cast<uint32_t*>(ptr), words);
  if (hipGetLastError() != hipSuccess) return W4A16_ERR_LAUNCH;
  g_scratch.emplace(dev, static_cast<char*>(ptr));
  *out = static_cast<char*>(ptr);
  return W4A16_OK;
}

// Workspace of one launch: the per-stream buffer, or (noalloc) the fixed scratch array,
// refused with W4A16_ERR_WORKSPACE when the plan needs more than it holds.
int launch_workspace(int dev, hipStream_t st, size_t counters, size_t floats, bool noalloc,
                     int** cnt, float** part) {
  if (!noalloc) return get_workspace(dev, st, counters, floats, cnt, part);
  *cnt = nullptr;
  *part = nullptr;
  if (counters == 0 && floats == 0) return W4A16_OK;
  if (counters * sizeof(int) > (size_t)W4A16_WS_COUNTER_BYTES ||
      floats * sizeof(float) > kScratchPartBytes)
    return W4A16_ERR_WORKSPACE;
  char* base = nullptr;
  int rc = scratch_for_device(dev, st, &base);
  if (rc) return rc;
  *cnt = reinterpret_cast<int*>(base);
  *part = reinterpret_cast<float*>(base + W4A16_WS_COUNTER_BYTES);
  return W4A16_OK;
}

// Weight format of a dense launch: zero-points or not, groups of 64 rows or not.
inline int dense_mode(bool asym, int group) {
  return group == 64 ? (asym ? W_ASYM64 : W_SYM64) : (asym ? W_ASYM : W_SYM);
}

inline int launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return W4A16_ERR_LAUNCH;
  }
  return W4A16_OK;
}

int run_skinny(int mode, const uint16_t* X, const void* w, const uint16_t* sp, const void* zp,
               uint16_t* Y, int M, int N, int K, int group, int variant, int splits,
               void* stream, const float* xscale = nullptr, bool noalloc = false) {
  SkinnyPlan plan;
  int rc = skinny_make_plan(M, N, K, group, mode, variant, splits, &plan);
  if (rc) return rc;
  int dev;
  if ((rc = check_device(&dev))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* cnt;
  float* part;
  if ((rc = launch_workspace(dev, st, plan.counters, plan.part_floats, noalloc, &cnt, &part)))
    return rc;
  return launched(skinny_launch(plan, X, w, sp, static_cast<const uint32_t*>(zp), Y, part, cnt,
                                M, N, K, group, st, xscale));
}

// Which kernel an automatic plan uses, from sweeps on MI355X: the skinny (memory-bound)
// kernel up to 32 rows; above that the tiled kernel (1.6-2.1x faster at M = 48-64 on
// layers of 70-235 Mi weights), except on layers under 32 Mi weights below 256 rows
// (1024 x 1024, 2560 x 2560, 3072 x 768, 4096 x 4096), where the tiled kernel has too few
// tiles and the skinny kernel with several row blocks fills the chip (2.2-2.6x faster
// than 16-row tiles on 1024 x 1024 and 3072 x 768 at M = 48-128).  The 2:4 format on
// layers of 128 Mi weights or more takes the tiled kernel's 32-row tiles from 17 rows on
// (1.16x over the skinny kernel at M = 32 on 8192 x 28672); up to 16 rows its skinny plan
// with eight column tiles per wave is 1.10x faster than 16-row tiles.
bool use_tiled(int M, int N, int K, int mode = W_SYM) {
  const long long kn = (long long)K * N;
  if (mode == W_SP24 && M > 16 && kn >= (128LL << 20)) return true;
  if (M <= 32) return false;
  if (M >= 256) return true;
  return kn >= (32LL << 20);
}

// MXFP4 automatic plan: the decode kernel up to 32 rows (measured 1.3-2.3x faster than
// 32-row tiles at M = 1-16 and 1.0-1.7x at M = 17-32 on the 7B/70B-class layers), except
// at 17-32 rows with 257-512 column tiles, where the 32-row tiles' shared X tile wins
// (1.05-1.12x on 28672 x 8192); the tiled kernel above.
bool mx_uses_decode(int M, int N) {
  const int tiles = N / 16;
  return M <= 32 && (M <= 16 || tiles <= 256 || tiles > 512);
}

int run_tiled(int mode, const uint16_t* X, const void* w, const uint16_t* sp, const void* zp,
              uint16_t* Y, int M, int N, int K, int variant, int grid, void* stream,
              const float* xscale = nullptr, bool noalloc = false) {
  TiledPlan plan;
  int rc = tiled_make_plan(M, N, K, mode, variant, grid, &plan);
  if (rc) return rc;
  int dev;
  if ((rc = check_device(&dev))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* cnt;
  float* part;
  if ((rc = launch_workspace(dev, st, 0, plan.part_floats, noalloc, &cnt, &part))) return rc;
  return launched(
      tiled_launch(plan, X, w, sp, static_cast<const uint32_t*>(zp), Y, part, st, xscale));
}

// bf16 and fp8 activations on the fp16 tiled kernel: the rows of X are rewritten in fp16
// (bf16: with a power-of-two scale each, exact within 2^32 of the row's maximum; fp8 E4M3:
// exactly, see bf16_rows.hip), then the dense fp16 tiled plan runs with the row scales
// applied to its fp32 sums (bf16: the inverse powers of two, and a bf16 store; fp8: the
// caller's scales, or none).  Workspace floats: [stream-K partials | row scales | fp16 rows],
// each part 256-byte aligned.
inline size_t round64(size_t n) { return (n + 63) / 64 * 64; }
// Automatic bf16 and fp8 plans: the skinny kernel up to 32 rows (and where w4a16_gemm keeps
// it), the fp16 tiled kernel on rewritten rows above.
bool uses_rows16(int M, int N, int K) { return use_tiled(M, N, K); }
size_t rows16_floats(const TiledPlan& t, int M, int K) {
  return round64(t.part_floats) + round64((size_t)M) + (size_t)M * K / 2;
}

enum RowsSource { ROWS_BF16, ROWS_FP8 };

int run_rows16(RowsSource src, int mode16, const void* X, const float* xscale, const void* w,
               const uint16_t* sp, const void* zp, uint16_t* Y, int M, int N, int K, int variant,
               int grid, void* stream) {
  TiledPlan plan;
  int rc = tiled_make_plan(M, N, K, mode16, variant, grid, &plan);
  if (rc) return rc;
  int dev;
  if ((rc = check_device(&dev))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int* cnt;
  float* part;
  if ((rc = get_workspace(dev, st, 0, rows16_floats(plan, M, K), &cnt, &part))) return rc;
  float* rscale = part + round64(plan.part_floats);
  uint16_t* xh = reinterpret_cast<uint16_t*>(rscale + round64((size_t)M));
  if (src == ROWS_BF16) {
    if ((rc = launched(launch_bf16_rows_to_f16(static_cast<const uint16_t*>(X), xh, rscale, M,
                                               K, st))))
      return rc;
    xscale = rscale;
  } else if ((rc = launched(launch_fp8_rows_to_f16(static_cast<const uint8_t*>(X), xh,
                                                   (size_t)M * K, st)))) {
    return rc;
  }
  return launched(tiled_launch(plan, xh, w, sp, static_cast<const uint32_t*>(zp), Y, part, st,
                               xscale, true, src == ROWS_BF16));
}

// Variant numbering of the ABI: the skinny variants first, then the tiled ones.
// For a tiled variant the `splits` argument is the number of persistent workgroups.
int run_fused(int mode, const uint16_t* X, const void* w, const uint16_t* sp, const void* zp,
              uint16_t* Y, int M, int N, int K, int group, int variant, int splits,
              void* stream, bool noalloc = false) {
  const int ns = skinny_variant_count();
  if (variant >= ns)
    return run_tiled(mode, X, w, sp, zp, Y, M, N, K, variant - ns, splits, stream, nullptr,
                     noalloc);
  if (variant < 0 && splits == 0 && use_tiled(M, N, K, mode)) {
    // shapes whose tiles would need buffer offsets past 2 GiB stay on the skinny kernel
    TiledPlan t;
    if (tiled_make_plan(M, N, K, mode, -1, 0, &t) == 0)
      return run_tiled(mode, X, w, sp, zp, Y, M, N, K, -1, 0, stream, nullptr, noalloc);
  }
  return run_skinny(mode, X, w, sp, zp, Y, M, N, K, group, variant, splits, stream, nullptr,
                    noalloc);
}

int check_gemm_args(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                    const uint16_t* Y, int M, int N, int K, int group) {
  if (!X || !wp || !sp || !Y) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (M <= 0) return W4A16_ERR_SHAPE;
  if ((long long)M * K > (1LL << 40) || (long long)M * N > (1LL << 40)) return W4A16_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(wp) || !aligned16(sp) || !aligned16(Y) ||
      (zp && !aligned16(zp)))
    return W4A16_ERR_ALIGN;
  return W4A16_OK;
}

}  // namespace

extern "C" {

int w4a16_layout_version(void) { return LAYOUT_VERSION; }

const char* w4a16_strerror(int code) {
  switch (code) {
    case W4A16_OK: return "success";
    case W4A16_ERR_NULL: return "a required pointer is NULL";
    case W4A16_ERR_SHAPE: return "invalid shape (M,N,K >= 1, K % 128 == 0, group 64 or a multiple of 128 dividing K, N % 16 == 0)";
    case W4A16_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case W4A16_ERR_DEVICE: return "no HIP device, or the current device is not gfx950";
    case W4A16_ERR_LAUNCH: return "kernel launch failed";
    case W4A16_ERR_WORKSPACE: return "workspace allocation failed";
    case W4A16_ERR_NOT24: return "weights are not 2:4 sparse along K";
    case W4A16_ERR_ARG: return "an enumerated argument is out of range";
    default: return "unknown error code";
  }
}

size_t w4a16_packed_bytes(int K, int N, int group, int which) {
  if (check_weight_shape(K, N, group)) return 0;
  const size_t KN = (size_t)K * N, Gk = (size_t)(K / KBLK), SH = group == 64 ? 2 : 1;
  const bool sparse_ok = group != 64;
  switch (which) {
    case W4A16_BUF_W: return KN / 2;
    case W4A16_BUF_S: return 2 * Gk * N * SH;
    case W4A16_BUF_Z: return Gk * N / 2 * SH;
    case W4A16_BUF_SPARSE_V: return sparse_ok ? KN / 4 : 0;
    case W4A16_BUF_SPARSE_I: return sparse_ok ? KN / 8 : 0;
    case W4A16_BUF_SPARSE_S: return sparse_ok ? 2 * Gk * N : 0;
    default: return 0;
  }
}

int w4a16_repack(const int32_t* q, const uint16_t* s, const int32_t* z, void* wp, uint16_t* sp,
                 void* zp, int K, int N, int group, void* stream) {
  if (!q || !s || !wp || !sp) return W4A16_ERR_NULL;
  if ((z == nullptr) != (zp == nullptr)) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(s) || !aligned16(wp) || !aligned16(sp) ||
      (z && (!aligned16(z) || !aligned16(zp))))
    return W4A16_ERR_ALIGN;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_repack(q, s, z, static_cast<uint32_t*>(wp), sp,
                                static_cast<uint32_t*>(zp), K, N, group,
                                static_cast<hipStream_t>(stream)));
}

int w4a16_unpack(const void* wp, const uint16_t* sp, const void* zp, int32_t* q, uint16_t* s,
                 int32_t* z, int K, int N, int group, void* stream) {
  if (!q || !s || !wp || !sp) return W4A16_ERR_NULL;
  if ((z == nullptr) != (zp == nullptr)) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(s) || !aligned16(wp) || !aligned16(sp) ||
      (z && (!aligned16(z) || !aligned16(zp))))
    return W4A16_ERR_ALIGN;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_unpack(static_cast<const uint32_t*>(wp), sp,
                                static_cast<const uint32_t*>(zp), q, s, z, K, N, group,
                                static_cast<hipStream_t>(stream)));
}

int w4a16_gemm(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
               uint16_t* Y, int M, int N, int K, int group, void* stream) {
  int rc = check_gemm_args(X, wp, sp, zp, Y, M, N, K, group);
  if (rc) return rc;
  return run_fused(dense_mode(zp != nullptr, group), X, wp, sp, zp, Y, M, N, K, group, -1, 0,
                   stream);
}

int w4a16_gemm_noalloc(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                       uint16_t* Y, int M, int N, int K, int group, void* stream) {
  int rc = check_gemm_args(X, wp, sp, zp, Y, M, N, K, group);
  if (rc) return rc;
  return run_fused(dense_mode(zp != nullptr, group), X, wp, sp, zp, Y, M, N, K, group, -1, 0,
                   stream, true);
}

int w4a16_gemm_plan(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                    uint16_t* Y, int M, int N, int K, int group, int variant, int splits,
                    void* stream) {
  int rc = check_gemm_args(X, wp, sp, zp, Y, M, N, K, group);
  if (rc) return rc;
  if (variant < -1 || variant >= w4a16_gemm_variants() || splits < 0) return W4A16_ERR_ARG;
  return run_fused(dense_mode(zp != nullptr, group), X, wp, sp, zp, Y, M, N, K, group, variant,
                   splits, stream);
}

int w4a16_gemm_variants(void) { return skinny_variant_count() + tiled_variant_count(W_SYM); }
const char* w4a16_gemm_variant_name(int variant) {
  const int ns = skinny_variant_count();
  return variant >= ns ? tiled_variant_name(W_SYM, variant - ns) : skinny_variant_name(variant);
}

int w4a16_gemm_describe(int M, int N, int K, int group, int* out4) {
  if (!out4) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (M <= 0) return W4A16_ERR_SHAPE;
  TiledPlan t;
  if (use_tiled(M, N, K) && tiled_make_plan(M, N, K, W_SYM, -1, 0, &t) == 0) {
    out4[0] = skinny_variant_count() + t.variant;
    out4[1] = t.args.grid;
    out4[2] = t.wgs;
    out4[3] = t.threads;
    return W4A16_OK;
  }
  SkinnyPlan p;
  if ((rc = skinny_make_plan(M, N, K, group, W_SYM, -1, 0, &p))) return rc;
  out4[0] = p.variant;
  out4[1] = p.splits;
  out4[2] = p.wgs;
  out4[3] = p.threads;
  return W4A16_OK;
}

size_t w4a16_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % KBLK != 0 || N % NTILE != 0) return 0;
  // the automatic plan of every weight format (the largest need), laid out as
  // get_workspace lays it out: counters rounded up to 64 ints, then the partials
  size_t need = 0;
  const int modes[] = {W_SYM, W_ASYM, W_SP24, W_FP16};
  for (int mode : modes) {
    size_t counters = 0, floats = 0;
    TiledPlan t;
    if (use_tiled(M, N, K, mode) && tiled_make_plan(M, N, K, mode, -1, 0, &t) == 0) {
      floats = t.part_floats;
    } else {
      SkinnyPlan p;
      if (skinny_make_plan(M, N, K, KBLK, mode, -1, 0, &p) != 0) continue;
      counters = (size_t)p.counters;
      floats = p.part_floats;
    }
    if (counters == 0 && floats == 0) continue;
    const size_t bytes = (counters + 63) / 64 * 64 * sizeof(int) + floats * sizeof(float);
    if (bytes > need) need = bytes;
  }
  // w4a16_gemm_bf16 and w4a8_gemm with groups of 64 run every M on the skinny kernel;
  // with larger groups they take the tiled kernel where w4a16_gemm does (their tiled plans
  // differ: fp8 needs an even number of 16-row tiles, bf16 has no eight-wave tiles)
  SkinnyPlan p;
  if (skinny_make_plan(M, N, K, KBLK, W_SYM8, -1, 0, &p) == 0) {
    const size_t bytes =
        ((size_t)p.counters + 63) / 64 * 64 * sizeof(int) + p.part_floats * sizeof(float);
    if ((p.counters || p.part_floats) && bytes > need) need = bytes;
  }
  TiledPlan t;
  if (skinny_make_plan(M, N, K, KBLK, W_SYMB, -1, 0, &p) == 0) {
    const size_t bytes =
        ((size_t)p.counters + 63) / 64 * 64 * sizeof(int) + p.part_floats * sizeof(float);
    if ((p.counters || p.part_floats) && bytes > need) need = bytes;
  }
  // w4a16_gemm_bf16 and w4a8_gemm above 32 rows: partials, row scales and the fp16 rows
  // (every group)
  for (int mode16 : {W_SYM, W_ASYM, W_SYM64, W_ASYM64}) {
    if (uses_rows16(M, N, K) && tiled_make_plan(M, N, K, mode16, -1, 0, &t) == 0) {
      const size_t bytes = rows16_floats(t, M, K) * sizeof(float);
      if (bytes > need) need = bytes;
    }
  }
  if (use_tiled(M, N, K) && tiled_make_plan(M, N, K, W_SYM8, -1, 0, &t) == 0) {
    const size_t bytes = t.part_floats * sizeof(float);
    if (bytes > need) need = bytes;
  }
  // w4a8_mx_gemm: the decode kernel needs none, the tiled kernel its stream-K partials
  if (!mx_uses_decode(M, N) && tiled_make_plan(M, N, K, W_MX4, -1, 0, &t) == 0) {
    const size_t bytes = t.part_floats * sizeof(float);
    if (bytes > need) need = bytes;
  }
  return need;
}

int w4a16_dequant(const int32_t* q, const uint16_t* s, const int32_t* z, uint16_t* Wt, int K,
                  int N, int group, void* stream) {
  if (!q || !s || !Wt) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(s) || !aligned16(Wt) || (z && !aligned16(z)))
    return W4A16_ERR_ALIGN;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_dequant(q, s, z, Wt, K, N, group, static_cast<hipStream_t>(stream)));
}

namespace {
int check_fp16_args(const uint16_t* X, const uint16_t* Wt, const uint16_t* Y, int M, int N,
                    int K) {
  if (!X || !Wt || !Y) return W4A16_ERR_NULL;
  if (M <= 0 || N <= 0 || K <= 0 || K % KBLK != 0 || N % NTILE != 0) return W4A16_ERR_SHAPE;
  if ((long long)N * K > (1LL << 40) || (long long)M * K > (1LL << 40) ||
      (long long)M * N > (1LL << 40))
    return W4A16_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(Wt) || !aligned16(Y)) return W4A16_ERR_ALIGN;
  return W4A16_OK;
}
}  // namespace

int w4a16_fp16_gemm(const uint16_t* X, const uint16_t* Wt, uint16_t* Y, int M, int N, int K,
                    void* stream) {
  int rc = check_fp16_args(X, Wt, Y, M, N, K);
  if (rc) return rc;
  return run_fused(W_FP16, X, Wt, nullptr, nullptr, Y, M, N, K, KBLK, -1, 0, stream);
}

int w4a16_fp16_gemm_variants(void) {
  return skinny_variant_count() + tiled_variant_count(W_FP16);
}
const char* w4a16_fp16_gemm_variant_name(int variant) {
  const int ns = skinny_variant_count();
  return variant >= ns ? tiled_variant_name(W_FP16, variant - ns) : skinny_variant_name(variant);
}

int w4a16_fp16_gemm_plan(const uint16_t* X, const uint16_t* Wt, uint16_t* Y, int M, int N, int K,
                         int variant, int splits, void* stream) {
  int rc = check_fp16_args(X, Wt, Y, M, N, K);
  if (rc) return rc;
  if (variant < -1 || variant >= w4a16_fp16_gemm_variants() || splits < 0) return W4A16_ERR_ARG;
  return run_fused(W_FP16, X, Wt, nullptr, nullptr, Y, M, N, K, KBLK, variant, splits, stream);
}

// ---- 2:4 structured sparsity ----------------------------------------------------------
namespace {
std::map<int, int*> g_bad;  // per-device counter of runs that are not 2:4
}

int w4a16_sparse24_repack(const int32_t* q, const uint16_t* s, void* vp, void* idx, uint16_t* sp,
                          int K, int N, int group, void* stream) {
  if (!q || !s || !vp || !idx || !sp) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (group == 64) return W4A16_ERR_SHAPE;  // 2:4 format: groups of 128 rows or more
  if (!aligned16(q) || !aligned16(s) || !aligned16(vp) || !aligned16(idx) || !aligned16(sp))
    return W4A16_ERR_ALIGN;
  int dev;
  if ((rc = check_device(&dev))) return rc;
  int* bad = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_bad.find(dev);
    if (it == g_bad.end()) {
      if (hipMalloc(&bad, sizeof(int)) != hipSuccess) {
        (void)hipGetLastError();
        return W4A16_ERR_WORKSPACE;
      }
      g_bad[dev] = bad;
    } else {
      bad = it->second;
    }
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = launched(launch_sparse_compress(q, s, static_cast<uint32_t*>(vp),
                                            static_cast<uint32_t*>(idx), sp, bad, K, N, group,
                                            st))))
    return rc;
  int h = 0;
  if (hipMemcpyAsync(&h, bad, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return W4A16_ERR_LAUNCH;
  }
  return h ? W4A16_ERR_NOT24 : W4A16_OK;
}

int w4a16_sparse24_unpack(const void* vp, const void* idx, const uint16_t* sp, int32_t* q,
                          uint16_t* s, int K, int N, int group, void* stream) {
  if (!q || !s || !vp || !idx || !sp) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, group);
  if (rc) return rc;
  if (group == 64) return W4A16_ERR_SHAPE;  // 2:4 format: groups of 128 rows or more
  if (!aligned16(q) || !aligned16(s) || !aligned16(vp) || !aligned16(idx) || !aligned16(sp))
    return W4A16_ERR_ALIGN;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_sparse_decompress(static_cast<const uint32_t*>(vp),
                                           static_cast<const uint32_t*>(idx), sp, q, s, K, N,
                                           group, static_cast<hipStream_t>(stream)));
}

int w4a16_sparse24_gemm(const uint16_t* X, const void* vp, const void* idx, const uint16_t* sp,
                        uint16_t* Y, int M, int N, int K, int group, void* stream) {
  if (!idx) return W4A16_ERR_NULL;
  int rc = check_gemm_args(X, vp, sp, idx, Y, M, N, K, group);
  if (rc) return rc;
  if (group == 64) return W4A16_ERR_SHAPE;
  return run_fused(W_SP24, X, vp, sp, idx, Y, M, N, K, group, -1, 0, stream);
}

int w4a16_sparse24_gemm_plan(const uint16_t* X, const void* vp, const void* idx,
                             const uint16_t* sp, uint16_t* Y, int M, int N, int K, int group,
                             int variant, int splits, void* stream) {
  if (!idx) return W4A16_ERR_NULL;
  int rc = check_gemm_args(X, vp, sp, idx, Y, M, N, K, group);
  if (rc) return rc;
  if (group == 64) return W4A16_ERR_SHAPE;
  if (variant < -1 || variant >= w4a16_gemm_variants() || splits < 0) return W4A16_ERR_ARG;
  return run_fused(W_SP24, X, vp, sp, idx, Y, M, N, K, group, variant, splits, stream);
}

}  // extern "C"

// ---- bf16 activations ----------------------------------------------------------------
namespace {
// "rows16_" + the fp16-path tiled variant's name, built once
const char* rows_variant_name(int v) {
  static const std::vector<std::string> names = [] {
    std::vector<std::string> n;
    for (int i = 0; i < tiled_variant_count(W_SYM); ++i)
      n.push_back(std::string("rows16_") + tiled_variant_name(W_SYM, i));
    return n;
  }();
  return v >= 0 && v < (int)names.size() ? names[v].c_str() : nullptr;
}
}  // namespace

int w4a16_gemm_bf16_variants(void) {
  return skinny_variant_count() + tiled_variant_count(W_SYMB) + tiled_variant_count(W_SYM);
}

const char* w4a16_gemm_bf16_variant_name(int variant) {
  const int ns = skinny_variant_count(), nb = tiled_variant_count(W_SYMB);
  if (variant < 0) return nullptr;
  if (variant < ns) return skinny_variant_name(variant);
  if (variant < ns + nb) return tiled_variant_name(W_SYMB, variant - ns);
  return rows_variant_name(variant - ns - nb);
}

int w4a16_gemm_bf16_plan(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                         uint16_t* Y, int M, int N, int K, int group, int variant, int splits,
                         void* stream) {
  int rc = check_gemm_args(X, wp, sp, zp, Y, M, N, K, group);
  if (rc) return rc;
  const int ns = skinny_variant_count(), nb = tiled_variant_count(W_SYMB);
  if (variant < -1 || variant >= w4a16_gemm_bf16_variants() || splits < 0) return W4A16_ERR_ARG;
  const int mode = group == 64 ? (zp ? W_ASYMB64 : W_SYMB64) : (zp ? W_ASYMB : W_SYMB);
  const int mode16 = dense_mode(zp != nullptr, group);
  // skinny variants first, then the bf16 tiled ones (w4a16_gemm_plan's numbering), then the
  // fp16 tiled ones on rewritten rows
  if (variant >= ns + nb)
    return run_rows16(ROWS_BF16, mode16, X, nullptr, wp, sp, zp, Y, M, N, K, variant - ns - nb,
                      splits, stream);
  if (variant >= ns) {
    if (group == 64) return W4A16_ERR_ARG;
    return run_tiled(mode, X, wp, sp, zp, Y, M, N, K, variant - ns, splits, stream);
  }
  if (variant < 0 && splits == 0 && uses_rows16(M, N, K)) {
    TiledPlan t;
    if (tiled_make_plan(M, N, K, mode16, -1, 0, &t) == 0)
      return run_rows16(ROWS_BF16, mode16, X, nullptr, wp, sp, zp, Y, M, N, K, -1, 0, stream);
  }
  return run_skinny(mode, X, wp, sp, zp, Y, M, N, K, group, variant, splits, stream);
}

int w4a16_gemm_bf16(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                    uint16_t* Y, int M, int N, int K, int group, void* stream) {
  return w4a16_gemm_bf16_plan(X, wp, sp, zp, Y, M, N, K, group, -1, 0, stream);
}

// ---- caller-owned workspace -----------------------------------------------------------
int w4a16_set_workspace(void* ptr, size_t bytes, void* stream) {
  if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return W4A16_ERR_ALIGN;
  if (ptr && bytes < (size_t)W4A16_WS_COUNTER_BYTES + 256) return W4A16_ERR_WORKSPACE;
  int dev;
  int rc = check_device(&dev);
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (capturing(st)) return W4A16_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_ws[std::make_pair(dev, st)];
  // the caller may free its old buffer once this returns: let launches on it drain first
  if (ws.ptr && ws.external && hipStreamSynchronize(st) != hipSuccess) {
    (void)hipGetLastError();
    return W4A16_ERR_LAUNCH;
  }
  // a library-owned buffer is kept, not freed (graphs captured earlier may use it)
  if (ws.ptr && !ws.external) g_retired.push_back(ws.ptr);
  ws = Workspace();
  if (!ptr) return W4A16_OK;
  if (hipMemsetAsync(ptr, 0, W4A16_WS_COUNTER_BYTES, st) != hipSuccess) {
    (void)hipGetLastError();
    return W4A16_ERR_LAUNCH;
  }
  ws.ptr = ptr;
  ws.external = true;
  ws.counter_ints = W4A16_WS_COUNTER_BYTES / sizeof(int);
  ws.part_floats = (bytes - W4A16_WS_COUNTER_BYTES) / sizeof(float);
  return W4A16_OK;
}

// ---- fp8 (E4M3) activations: W4A8 ------------------------------------------------------
int w4a8_gemm_plan(const uint8_t* X8, const float* xscale, const void* wp, const uint16_t* sp,
                   const void* zp, uint16_t* Y, int M, int N, int K, int group, int variant,
                   int splits, void* stream) {
  const uint16_t* X = reinterpret_cast<const uint16_t*>(X8);
  int rc = check_gemm_args(X, wp, sp, zp, Y, M, N, K, group);
  if (rc) return rc;
  if (xscale && (reinterpret_cast<uintptr_t>(xscale) & 3u) != 0) return W4A16_ERR_ALIGN;
  if (variant < -1 || variant >= w4a16_gemm_bf16_variants() || splits < 0) return W4A16_ERR_ARG;
  const int mode = group == 64 ? (zp ? W_ASYM8G64 : W_SYM8G64) : (zp ? W_ASYM8 : W_SYM8);
  const int mode16 = dense_mode(zp != nullptr, group);
  // numbered like w4a16_gemm_bf16_plan: the skinny variants, the fp8 tiled ones (groups of
  // 128 rows or more), then the fp16 tiled ones on rewritten rows (every group)
  const int ns = skinny_variant_count(), nt = tiled_variant_count(W_SYM8);
  if (variant >= ns + nt)
    return run_rows16(ROWS_FP8, mode16, X8, xscale, wp, sp, zp, Y, M, N, K, variant - ns - nt,
                      splits, stream);
  if (variant >= ns)
    return run_tiled(mode, X, wp, sp, zp, Y, M, N, K, variant - ns, splits, stream, xscale);
  if (variant < 0 && splits == 0 && uses_rows16(M, N, K)) {
    TiledPlan t;
    if (tiled_make_plan(M, N, K, mode16, -1, 0, &t) == 0)
      return run_rows16(ROWS_FP8, mode16, X8, xscale, wp, sp, zp, Y, M, N, K, -1, 0, stream);
  }
  return run_skinny(mode, X, wp, sp, zp, Y, M, N, K, group, variant, splits, stream, xscale);
}

int w4a8_gemm(const uint8_t* X8, const float* xscale, const void* wp, const uint16_t* sp,
              const void* zp, uint16_t* Y, int M, int N, int K, int group, void* stream) {
  return w4a8_gemm_plan(X8, xscale, wp, sp, zp, Y, M, N, K, group, -1, 0, stream);
}

// ---- MXFP4 weights x fp8 activations: scales applied inside the matrix instruction ----
// decode kernel taken by the automatic plan at M <= 32 (index among the decode variants:
// 1, 2 or 4 column tiles per workgroup).  Measured on the 7B/70B-class layers: one tile
// (the most workgroups) is best or within 6% at M <= 8 and wherever N <= 4096, except at
// 2-8 rows on layers of more than 1024 column tiles (8192 x 28672: four tiles 1.14x faster
// at M = 8); at M = 9-32 more columns per workgroup cut the re-reads of X from L2: two
// tiles for N <= 8192 (512 tiles), four above (1.1-1.4x over one tile on 4096 x 12288,
// 8192 x 10240, 8192 x 28672).
static int mx_decode_default(int M, int N) {
  const int tiles = N / 16;
  if (M <= 8) return M > 1 && tiles > 1024 ? 2 : 0;
  if (tiles <= 256) return 0;
  return tiles <= 512 ? 1 : 2;
}

int w4a8_mx_repack(const int32_t* q, const uint8_t* e, void* wp, void* sp, int K, int N,
                   void* stream) {
  if (!q || !e || !wp || !sp) return W4A16_ERR_NULL;
  int rc = check_weight_shape(K, N, KBLK);
  if (rc) return rc;
  if (!aligned16(q) || !aligned16(wp) || !aligned16(sp)) return W4A16_ERR_ALIGN;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_mx_repack(q, e, static_cast<uint32_t*>(wp), static_cast<uint8_t*>(sp),
                                   K, N, static_cast<hipStream_t>(stream)));
}

int w4a8_mx_gemm_plan(const uint8_t* X8, const float* xscale, const void* wp, const void* sp,
                      uint16_t* Y, int M, int N, int K, int variant, int grid, void* stream) {
  const uint16_t* X = reinterpret_cast<const uint16_t*>(X8);
  const uint16_t* S = static_cast<const uint16_t*>(sp);
  int rc = check_gemm_args(X, wp, S, nullptr, Y, M, N, K, KBLK);
  if (rc) return rc;
  if (xscale && (reinterpret_cast<uintptr_t>(xscale) & 3u) != 0) return W4A16_ERR_ALIGN;
  const int nt = tiled_variant_count(W_MX4);
  if (variant < -1 || variant >= nt + mx_decode_variant_count() || grid < 0) return W4A16_ERR_ARG;
  if (variant < 0 && grid == 0 && mx_uses_decode(M, N)) variant = nt + mx_decode_default(M, N);
  if (variant >= nt) {
    if (M > 32) return W4A16_ERR_ARG;
    int dev;
    if ((rc = check_device(&dev))) return rc;
    return launched(mx_decode_launch(variant - nt, X8, xscale, wp, static_cast<const uint8_t*>(sp),
                                     Y, M, N, K, static_cast<hipStream_t>(stream)));
  }
  return run_tiled(W_MX4, X, wp, S, nullptr, Y, M, N, K, variant, grid, stream, xscale);
}

int w4a8_mx_variants(void) { return tiled_variant_count(W_MX4) + mx_decode_variant_count(); }
const char* w4a8_mx_variant_name(int variant) {
  const int nt = tiled_variant_count(W_MX4);
  return variant >= nt ? mx_decode_variant_name(variant - nt) : tiled_variant_name(W_MX4, variant);
}

int w4a8_mx_gemm(const uint8_t* X8, const float* xscale, const void* wp, const void* sp,
                 uint16_t* Y, int M, int N, int K, void* stream) {
  return w4a8_mx_gemm_plan(X8, xscale, wp, sp, Y, M, N, K, -1, 0, stream);
}

// ---- calibration kernels -------------------------------------------------------------
int w4a16_probe_read(const void* p, size_t bytes, uint32_t* out, void* stream) {
  if (!p || !out) return W4A16_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0) return W4A16_ERR_SHAPE;
  if (!aligned16(p)) return W4A16_ERR_ALIGN;
  int rc;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_probe_read(p, bytes, out, static_cast<hipStream_t>(stream)));
}

int w4a16_probe_mfma(int workgroups, int iters, float* out, void* stream) {
  if (!out) return W4A16_ERR_NULL;
  if (workgroups < 1 || workgroups > 65536 || iters < 1) return W4A16_ERR_ARG;
  int rc;
  if ((rc = check_device(nullptr))) return rc;
  return launched(launch_probe_mfma(workgroups, iters, out, static_cast<hipStream_t>(stream)));
}

double w4a16_probe_mfma_flops(int workgroups, int iters) {
  if (workgroups < 1 || iters < 1) return 0.0;
  return probe_mfma_flops(workgroups, iters);
}
