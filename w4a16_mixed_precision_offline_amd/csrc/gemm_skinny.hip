// Fused W4A16 GEMM for gfx950: Y[M,N] = X[M,K] * ((q - z) * s), plus the fp16
// baseline GEMM that shares its skeleton.
//
// What the pages ask of the fused kernel (Marlin; dingiv.github.io "Marlin",
// sections "反量化与 GEMM 融合", "Striped 划分与流水线", "反量化精度权衡";
// brain.gartu.xyz "Marlin / GPTQ-Marlin", "Architecture générale" and "Les 4
// innovations clés"; vecbase.com "Marlin Project Overview", "Key Techniques"):
//   * packed weights are read from memory once and turned into fp16 in
//     registers right before the matrix instruction; nothing dequantized is
//     written back;
//   * 4-bit -> fp16 is exact; products accumulate in fp32; Y is fp16;
//   * weight loads are issued ahead of use so that memory latency hides behind
//     compute; activations stay close (L2 / registers) and are reused;
//   * several warps of a block compute partial sums of the same output tile;
//   * the work is split so that every compute unit is busy for any shape, with
//     as few global reduction steps as possible.
//
// How this kernel maps that onto CDNA4 (own design):
//   * One wave owns NT tiles of 16 columns and MT tiles of 16 rows.  A 128-row
//     k-block of one tile is 1 KiB of packed codes in the repacked layout, one
//     16-byte non-temporal load per lane (see internal.h).
//   * Dequantization uses the 0x6400 exponent trick: OR-ing a nibble into the
//     mantissa of 1024.0 gives the exact fp16 1024+q (or 1024+16q for the high
//     nibble of a byte), and one packed fp16 add / fma removes the offset and the
//     zero-point, giving the exact integer q - z.  The scale is applied after the
//     four v_mfma_f32_16x16x32_f16 of the k-block, in fp32, on the 4 accumulators
//     of the lane (1 fma per output instead of 1 multiply per weight).
//   * The WK waves of a workgroup take interleaved k-blocks of the same output
//     tile and reduce through LDS in a fixed order.
//   * When a tile's K range is cut into `splits` slices owned by different
//     workgroups, each writes an fp32 partial, bumps an arrival counter, and the
//     last to arrive sums the slices in slice order (deterministic) and writes
//     Y; it also resets the counter for the next launch, so no memset is needed.
//   * Weight registers are double-buffered: the next k-block's loads are in
//     flight while the current one is dequantized and multiplied.
#include "internal.h"

namespace w4a16 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte loads: streamed (non-temporal) for weights, cached for activations
__device__ __forceinline__ u32x4 load16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}


// 8 codes of one repacked word -> 8 exact fp16 (q - z), in row order 0..7.
// c0 = -(1024 + z) and c1 = -(64 + z) in both halves.
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v c0, half2v c1) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const uint32_t t0 = (w & 0x000F000Fu) | 0x64006400u;   // 1024+q0 | 1024+q1
  const uint32_t t1 = (w & 0x00F000F0u) | 0x64006400u;   // 1024+16q2 | 1024+16q3
  const uint32_t t2 = (w8 & 0x000F000Fu) | 0x64006400u;  // 1024+q4 | 1024+q5
  const uint32_t t3 = (w8 & 0x00F000F0u) | 0x64006400u;  // 1024+16q6 | 1024+16q7
  const half2v h0 = __builtin_bit_cast(half2v, t0) + c0;
  const half2v h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, t1), sixteenth, c1);
  const half2v h2 = __builtin_bit_cast(half2v, t2) + c0;
  const half2v h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, t3), sixteenth, c1);
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

template <int MT, int NT, int MODE>
struct Stage {
  u32x4 w[NT][MODE == W_FP16 ? 4 : 1];  // packed codes (or fp16 rows for the baseline)
  uint32_t s[NT];                       // fp16 scale bits of the lane's column
  uint2 z[NT];                          // 16 zero-points of the tile (ASYM)
  u32x4 x[MT][4];                       // X fragments for the four 32-row steps
};

template <int MT, int NT, int MODE>
__device__ __forceinline__ void load_stage(Stage<MT, NT, MODE>& S, int kb, int lane, int t0,
                                           int Gk, int G, int gpb, int K,
                                           const uint4* __restrict__ W,
                                           const uint16_t* __restrict__ Sp,
                                           const uint2* __restrict__ Zp,
                                           const uint16_t* const xrow[MT], const bool xok[MT]) {
  const int g = kb / gpb;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (MODE == W_FP16) {
      // baseline: W is fp16 [N][K]; the lane's column n, rows 32j + 8(lane/16) + 0..7
      const uint16_t* row = reinterpret_cast<const uint16_t*>(W) +
                            (long)((t0 + t) * 16 + (lane & 15)) * K + kb * KBLK + 8 * (lane >> 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) S.w[t][j] = load16_nt(row + 32 * j);
    } else {
      S.w[t][0] = load16_nt(W + ((long)(t0 + t) * Gk + kb) * 64 + lane);
      S.s[t] = Sp[((long)(t0 + t) * G + g) * 16 + (lane & 15)];
      if (MODE == W_ASYM) S.z[t] = Zp[(long)(t0 + t) * G + g];
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint16_t* p = xrow[mt] + kb * KBLK;
#pragma unroll
    for (int j = 0; j < 4; ++j) S.x[mt][j] = xok[mt] ? load16(p + 32 * j) : u32x4{0, 0, 0, 0};
  }
}

template <int MT, int NT, int MODE>
__device__ __forceinline__ void compute_stage(const Stage<MT, NT, MODE>& S, float4v (&acc)[NT][MT],
                                              int lane, int mtiles_live) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    half8 b[4];
    if (MODE == W_FP16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = __builtin_bit_cast(half8, S.w[t][j]);
    } else {
      half2v c0, c1;
      if (MODE == W_ASYM) {
        const int c = lane & 15;
        const uint32_t zw = c < 8 ? S.z[t].x : S.z[t].y;
        const int zq = (int)((zw >> (4 * (c & 7))) & 15u);
        const _Float16 a0 = (_Float16)(float)(-1024 - zq);
        const _Float16 a1 = (_Float16)(float)(-64 - zq);
        c0 = half2v{a0, a0};
        c1 = half2v{a1, a1};
      } else {
        c0 = half2v{(_Float16)-1032.0f, (_Float16)-1032.0f};
        c1 = half2v{(_Float16)-72.0f, (_Float16)-72.0f};
      }
      b[0] = dequant_word(S.w[t][0].x, c0, c1);
      b[1] = dequant_word(S.w[t][0].y, c0, c1);
      b[2] = dequant_word(S.w[t][0].z, c0, c1);
      b[3] = dequant_word(S.w[t][0].w, c0, c1);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mtiles_live) {
        if (MODE == W_FP16) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                __builtin_bit_cast(half8, S.x[mt][j]), b[j], acc[t][mt], 0, 0, 0);
        } else {
          float4v g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j)
            g = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, S.x[mt][j]),
                                                       b[j], g, 0, 0, 0);
          const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)S.s[t]);
          acc[t][mt] += sc * g;
        }
      }
    }
  }
}

// Split-K hand-off between workgroups on different XCDs.  Each XCD has its own
// L2, so ordinary stores may sit in one L2 while another XCD reads stale data.
// Relaxed agent-scope atomic loads and stores compile to sc1 accesses, which are
// coherent across XCDs by themselves; what an agent-scope release/acquire adds on
// top (an L2 write-back / invalidate) is only needed for ordinary accesses and is
// expensive.  So partials are written and read exclusively with sc1 accesses, and
// the release is "all sc1 stores complete (s_waitcnt vmcnt(0)) before the counter
// increment"; the acquire is "partials are read only after the increment returned".
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int NT, int WK, int D, int MODE>
__global__ __launch_bounds__(64 * WK) void skinny_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ W, const uint16_t* __restrict__ Sp,
    const uint2* __restrict__ Zp, uint16_t* __restrict__ Y, float* __restrict__ part,
    int* __restrict__ counters, int M, int N, int K, int gpb, int splits, int nblocks) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int bid = blockIdx.x;
  const int sl = bid % splits;
  bid /= splits;
  const int nb = bid % nblocks;
  const int mb = bid / nblocks;
  const int Gk = K / KBLK;
  const int G = Gk / gpb;
  // K range of this workgroup's slice, then this wave's contiguous chunk of it
  const int kb0 = (int)(((long)Gk * sl) / splits);
  const int kb1 = (int)(((long)Gk * (sl + 1)) / splits);
  const int nk_wg = kb1 - kb0;
  const int kw0 = kb0 + (nk_wg * wave) / WK;
  const int nk = kb0 + (nk_wg * (wave + 1)) / WK - kw0;
  const int t0 = nb * NT;
  const int m0 = mb * MT * 16;
  int mtiles_live = (M - m0 + 15) / 16;
  if (mtiles_live > MT) mtiles_live = MT;

  const uint16_t* xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = m0 + mt * 16 + (lane & 15);
    xok[mt] = r < M;
    xrow[mt] = X + (long)(xok[mt] ? r : 0) * K + 8 * (lane >> 4);
  }

  float4v acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = float4v{0.f, 0.f, 0.f, 0.f};

  // register ring of D stages: D k-blocks in flight ahead of the one being computed
  Stage<MT, NT, MODE> S[D];
#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nk) load_stage(S[d], kw0 + d, lane, t0, Gk, G, gpb, K, W, Sp, Zp, xrow, xok);
  for (int i = 0; i < nk; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (i + d < nk) {
        compute_stage(S[d], acc, lane, mtiles_live);
        if (i + d + D < nk)
          load_stage(S[d], kw0 + i + d + D, lane, t0, Gk, G, gpb, K, W, Sp, Zp, xrow, xok);
      }
    }
  }

  // ---- in-workgroup reduction over the WK waves, fixed order 0, 1, ..., WK-1 ----
  constexpr int NACC = NT * MT * 4;
  if (WK > 1) {
    __shared__ float4v red[(WK > 1 ? WK - 1 : 1) * 64 * NT * MT];  // [wave-1][lane][t][mt]
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[((wave - 1) * 64 + lane) * NT * MT + t * MT + mt] = acc[t][mt];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WK; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] += red[((w - 1) * 64 + lane) * NT * MT + t * MT + mt];
  }

  // ---- split-K: coherent partial, arrival counter, last arriver sums in slice order ----
  if (splits > 1) {
    const long tile_id = (long)mb * nblocks + nb;
    float* mypart = part + (tile_id * splits + sl) * (NACC * 64);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store_coherent(mypart + ((t * MT + mt) * 4 + r) * 64 + lane, acc[t][mt][r]);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // every sc1 store of this wave has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    int old = 0;
    if (lane == 0)
      old = __hip_atomic_fetch_add(counters + tile_id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __shfl(old, 0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (old != splits - 1) return;
    const float* base = part + tile_id * splits * (NACC * 64);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = 0.f;
          for (int s2 = 0; s2 < splits; ++s2)
            v += load_coherent(base + (long)s2 * (NACC * 64) + ((t * MT + mt) * 4 + r) * 64 + lane);
          acc[t][mt][r] = v;
        }
    if (lane == 0)
      __hip_atomic_store(counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+r of each m-tile, column lane%16 ----
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + mt * 16 + 4 * (lane >> 4) + r;
        const int col = (t0 + t) * 16 + (lane & 15);
        if (row < M)
          Y[(long)row * N + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[t][mt][r]);
      }
}

typedef void (*KernelFn)(const uint16_t*, const uint4*, const uint16_t*, const uint2*, uint16_t*,
                         float*, int*, int, int, int, int, int, int);

struct Variant {
  int MT, NT, WK, D;
  KernelFn sym, asym, f16;
  const char* name;
};

#define W4A16_VARIANT(MT, NT, WK, D)                                                     \
  Variant {                                                                              \
    MT, NT, WK, D, skinny_kernel<MT, NT, WK, D, W_SYM>, skinny_kernel<MT, NT, WK, D, W_ASYM>, \
        skinny_kernel<MT, NT, WK, D, W_FP16>,                                            \
        "skinny_mt" #MT "_nt" #NT "_wk" #WK "_d" #D                                      \
  }

const Variant kVariants[] = {
    W4A16_VARIANT(1, 1, 16, 2), W4A16_VARIANT(1, 1, 8, 2), W4A16_VARIANT(1, 1, 8, 4),
    W4A16_VARIANT(1, 1, 4, 4),  W4A16_VARIANT(1, 2, 8, 2), W4A16_VARIANT(1, 2, 4, 4),
    W4A16_VARIANT(1, 2, 16, 2), W4A16_VARIANT(2, 1, 8, 2), W4A16_VARIANT(2, 1, 16, 2),
    W4A16_VARIANT(2, 2, 8, 2),  W4A16_VARIANT(2, 1, 4, 4), W4A16_VARIANT(4, 1, 4, 2),
    W4A16_VARIANT(4, 1, 8, 2),  W4A16_VARIANT(4, 2, 4, 2),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int find_variant(int MT, int NT, int WK, int D) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].MT == MT && kVariants[i].NT == NT && kVariants[i].WK == WK &&
        kVariants[i].D == D)
      return i;
  return -1;
}

}  // namespace

int skinny_variant_count() { return kNumVariants; }
const char* skinny_variant_name(int v) {
  return (v >= 0 && v < kNumVariants) ? kVariants[v].name : nullptr;
}

int skinny_make_plan(int M, int N, int K, int group, int mode, int variant, int splits,
                     SkinnyPlan* p) {
  (void)group;
  if (variant < 0) {
    // measured on MI355X over the decode shapes: 16 waves per 16-column tile while the
    // tiles alone fill the 256 compute units, else two tiles per wave to halve the
    // activation loads per weight byte
    const long tiles = N / 16;
    const bool few = tiles <= 256;
    if (M <= 16)
      variant = few ? find_variant(1, 1, 16, 2)
                    : (N % 32 == 0 ? find_variant(1, 2, 8, 2) : find_variant(1, 1, 4, 4));
    else if (M <= 32)
      variant = (few || N % 32) ? find_variant(2, 1, 8, 2) : find_variant(2, 2, 8, 2);
    else
      variant = find_variant(4, 1, 8, 2);
  }
  if (variant < 0 || variant >= kNumVariants) return -8;
  const Variant& v = kVariants[variant];
  if (N % (16 * v.NT) != 0) return -2;
  const int Gk = K / KBLK;
  p->variant = variant;
  p->mode = mode;
  p->MT = v.MT;
  p->NT = v.NT;
  p->WK = v.WK;
  p->mblocks = (M + 16 * v.MT - 1) / (16 * v.MT);
  p->nblocks = N / (16 * v.NT);
  int maxs = Gk / v.WK;
  if (maxs < 1) maxs = 1;
  if (splits <= 0) {
    // split K only when the column tiles cannot give every compute unit a workgroup
    const long base = (long)p->mblocks * p->nblocks;
    const long target = 256;
    long sp = (target + base - 1) / base;
    splits = (int)(sp < 1 ? 1 : sp);
  }
  if (splits > maxs) splits = maxs;
  if (splits < 1) splits = 1;
  p->splits = splits;
  p->wgs = p->mblocks * p->nblocks * splits;
  p->threads = 64 * v.WK;
  p->part_floats = splits > 1 ? (size_t)p->mblocks * p->nblocks * splits * v.NT * v.MT * 256 : 0;
  p->counters = splits > 1 ? p->mblocks * p->nblocks : 0;
  return 0;
}

hipError_t skinny_launch(const SkinnyPlan& p, const uint16_t* X, const void* w,
                         const uint16_t* sp, const uint32_t* zp, uint16_t* Y, float* part,
                         int* counters, int M, int N, int K, int group, hipStream_t st) {
  const Variant& v = kVariants[p.variant];
  KernelFn fn = p.mode == W_FP16 ? v.f16 : (p.mode == W_ASYM ? v.asym : v.sym);
  hipLaunchKernelGGL(fn, dim3(p.wgs), dim3(p.threads), 0, st, X,
                     reinterpret_cast<const uint4*>(w), sp, reinterpret_cast<const uint2*>(zp), Y,
                     part, counters, M, N, K, group / KBLK, p.splits, p.nblocks);
  return hipGetLastError();
}

}  // namespace w4a16
