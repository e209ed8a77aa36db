// Fused W4A16 GEMM for larger M (prefill-sized batches) on gfx950:
// Y[M,N] = X[M,K] * ((q - z) * s), with the weights in the repacked layout.
//
// The pages' points that matter once M is large (dingiv.github.io "Marlin",
// sections "Striped 划分与流水线" and "反量化与 GEMM 融合"; vecbase.com "Marlin
// Project Overview", "Key Techniques"):
//   * the weight tile of a workgroup is unpacked in registers right before the
//     matrix instructions and reused for every activation row of the tile;
//   * the (tile, k-slice) work is cut into equal contiguous stripes, one per
//     persistent workgroup, so that every compute unit gets the same amount of
//     work for any number of tiles; tiles cut by a stripe boundary are summed
//     across workgroups in a second step.
//
// CDNA4 mapping (own design):
//   * A workgroup of 4 waves owns a tile of BM = 16*MT rows of Y by BN = 4*16*NTW
//     columns; the waves split the columns (wave w: 16*NTW columns) and share the
//     rows, so each weight byte is loaded and unpacked by exactly one wave, and
//     the activation tile is shared through LDS.
//   * Per 128-row k-block the activation tile (BM x 128 fp16) is loaded row-
//     contiguously (16 threads per 256-byte row) into registers and written into
//     one of two LDS buffers (rows padded to 272 bytes); a wave reads MFMA
//     fragments from it (lane l: row 16i + l%16, 8 halves at 32j + 8(l/16)).
//   * The weights of a wave's column tiles arrive as one 16-byte load per lane
//     per 1 KiB repacked block, which is already the operand fragment of the four
//     v_mfma_f32_16x16x32_f16 of the block.  Codes become exact fp16 (q - z) with
//     the 0x6400 exponent trick and are multiplied by the fp16 scale (one
//     rounding of W, as in the dequantized fp16 weight), so the accumulators need
//     no per-block rescaling.
//   * W is the MFMA's A operand and X its B operand: a lane's accumulator then
//     holds four consecutive columns of one row of Y (one 8-byte store).
//   * Loads for k-block kb+2 are issued while kb is computed (two register stages
//     for the weights, LDS double buffer for the activations).
//   * Work split: the first full rounds of tiles are handed out data-parallel (one
//     tile per workgroup per round, full K); the remaining tiles' (tile, k-block)
//     units are cut into equal contiguous stripes over all workgroups (stream-K).
//     A tile cut by a stripe boundary is finished by the last of its pieces to
//     arrive: every piece writes its fp32 partial with cross-XCD coherent (sc1)
//     stores and bumps the tile's arrival counter; the last arriver reads all
//     pieces back in stripe order (a fixed order, hence deterministic results),
//     writes Y and resets the counter for the next launch.
#include "internal.h"

namespace w4a16 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
// cache-policy bits of buffer instructions on gfx950
constexpr int kNT = 2;    // streamed (non-temporal)
constexpr int kSC1 = 16;  // coherent across the XCDs' L2s (relaxed agent-scope access)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}

__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

// 8 codes of one repacked word -> 8 fp16 weights RNE((q - z) * s), rows 0..7.
// c0 = -(1024 + z), c1 = -(64 + z), s2 = the scale in both halves.
__device__ __forceinline__ half8 dequant_scaled(uint32_t w, half2v c0, half2v c1, half2v s2,
                                                uint32_t magic) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const uint32_t t0 = and_or(w, 0x000F000Fu, magic);   // 1024+q0 | 1024+q1
  const uint32_t t1 = and_or(w, 0x00F000F0u, magic);   // 1024+16q2 | 1024+16q3
  const uint32_t t2 = and_or(w8, 0x000F000Fu, magic);  // 1024+q4 | 1024+q5
  const uint32_t t3 = and_or(w8, 0x00F000F0u, magic);  // 1024+16q6 | 1024+16q7
  // exact q - z, then one rounding of the product with the scale
  const half2v h0 = (__builtin_bit_cast(half2v, t0) + c0) * s2;
  const half2v h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, t1), sixteenth, c1) * s2;
  const half2v h2 = (__builtin_bit_cast(half2v, t2) + c0) * s2;
  const half2v h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, t3), sixteenth, c1) * s2;
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

constexpr int XSTRIDE = 272;  // bytes per activation row in LDS (256 + 16 against bank conflicts)
constexpr int WAVES = 4;

// Weights of one k-block for the NTW column tiles of a wave.
template <int NTW, int MODE>
struct WStage {
  u32x4 w[NTW];
  uint16_t s[NTW];
  uint2 z[NTW];
};

// Per-wave view of the current tile's weights: resources cover the wave's valid
// column tiles; the per-lane offsets hold the column-tile part of the address
// (kOutOfRange for tiles past N, which then read zeros), the scalar offset the
// k-block part.
template <int NTW>
struct WRsrc {
  rsrc_t w, s, z;
  uint32_t wo[NTW], so[NTW], zo[NTW];
};

template <int NTW, int MODE>
__device__ __forceinline__ void load_w(WStage<NTW, MODE>& S, const WRsrc<NTW>& R, int kb) {
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    S.w[t] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.w, R.wo[t], (uint32_t)kb * 1024u, kNT));
    S.s[t] = __builtin_amdgcn_raw_buffer_load_b16(R.s, R.so[t], (uint32_t)kb * 32u, 0);
    if (MODE == W_ASYM)
      S.z[t] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(R.z, R.zo[t], (uint32_t)kb * 8u, 0));
  }
}

// Activation rows of one k-block: thread tid loads rows tid/16 + 16c, bytes
// 16(tid%16) .. +15 of the block's 256 bytes.
template <int MT>
__device__ __forceinline__ void load_x(u32x4 (&xr)[MT], rsrc_t rx, const uint32_t (&xoff)[MT],
                                       int kb) {
#pragma unroll
  for (int c = 0; c < MT; ++c)
    xr[c] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff[c], (uint32_t)kb * 256u, 0));
}

template <int MT>
__device__ __forceinline__ void store_x(char* buf, const u32x4 (&xr)[MT], int tid) {
#pragma unroll
  for (int c = 0; c < MT; ++c)
    *reinterpret_cast<u32x4*>(buf + ((tid >> 4) + 16 * c) * XSTRIDE + (tid & 15) * 16) = xr[c];
}

// One k-block: 4 k-steps of 32; per step the wave unpacks its NTW weight
// fragments once and runs them against the MT activation fragments.
template <int MT, int NTW, int MODE>
__device__ __forceinline__ void compute_kblock(const char* buf, const WStage<NTW, MODE>& S,
                                               float4v (&acc)[MT][NTW], int lane, uint32_t magic) {
  half2v c0[NTW], c1[NTW], s2[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    int zq = 8;
    if (MODE == W_ASYM) {
      const int c = lane & 15;
      const uint32_t zw = c < 8 ? S.z[t].x : S.z[t].y;
      zq = (int)((zw >> (4 * (c & 7))) & 15u);
    }
    const _Float16 a0 = (_Float16)(float)(-1024 - zq);
    const _Float16 a1 = (_Float16)(float)(-64 - zq);
    c0[t] = half2v{a0, a0};
    c1[t] = half2v{a1, a1};
    const _Float16 sc = __builtin_bit_cast(_Float16, S.s[t]);
    s2[t] = half2v{sc, sc};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    half8 b[NTW];
#pragma unroll
    for (int t = 0; t < NTW; ++t) b[t] = dequant_scaled(S.w[t][j], c0[t], c1[t], s2[t], magic);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const half8 a = *reinterpret_cast<const half8*>(buf + (16 * i + (lane & 15)) * XSTRIDE +
                                                      64 * j + 16 * (lane >> 4));
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[t], a, acc[i][t], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Tile index -> (row tile, column tile), rows grouped by `group_m` so that the
// workgroups running at the same time share activation rows and weight columns.
__device__ __forceinline__ void tile_coords(int tt, int tiles_m, int tiles_n, int group_m, int& tm,
                                            int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = tt / per_group;
  const int first = g * group_m;
  const int gm = tiles_m - first < group_m ? tiles_m - first : group_m;
  const int r = tt - g * per_group;
  tm = first + r % gm;
  tn = r / gm;
}

template <int MT, int NTW, int MODE>
__global__ __launch_bounds__(64 * WAVES) void tiled_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ W,
    const uint16_t* __restrict__ Sp, const uint32_t* __restrict__ Zp, uint16_t* __restrict__ Y,
    float* __restrict__ part, int* __restrict__ counters, TiledArgs a) {
  constexpr int BM = 16 * MT;
  constexpr int BN = WAVES * 16 * NTW;
  constexpr int XBUF = BM * XSTRIDE;
  constexpr int PIECE = BM * BN;  // floats of one partial tile
  __shared__ __attribute__((aligned(16))) char lds[2 * XBUF];
  __shared__ int s_old;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Gk = a.K / KBLK;
  const int ntiles16 = a.N / 16;
  const uint32_t magic = 0x64006400u;

  // logical workgroup index: consecutive indices on one XCD (the hardware deals
  // workgroups to the 8 XCDs round-robin)
  int w = blockIdx.x;
  if (a.grid % 8 == 0) w = (blockIdx.x % 8) * (a.grid / 8) + blockIdx.x / 8;

  // ---- one segment: tile tt, k-blocks [kb0, kb1) ----
  auto run_segment = [&](int tt, int kb0, int kb1, float4v (&acc)[MT][NTW]) {
    int tm, tn;
    tile_coords(tt, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    const int m0 = tm * BM;
    const int rows = a.M - m0 < BM ? a.M - m0 : BM;
    const rsrc_t rx = make_rsrc(X + (size_t)m0 * a.K, (uint32_t)((size_t)rows * a.K * 2));
    uint32_t xoff[MT];
#pragma unroll
    for (int c = 0; c < MT; ++c) {
      const int r = (tid >> 4) + 16 * c;
      xoff[c] = r < rows ? (uint32_t)(((size_t)r * a.K + 8 * (tid & 15)) * 2) : kOutOfRange;
    }
    const int t_first = tn * (BN / 16) + wave * NTW;  // first 16-column tile of this wave
    int nvalid = ntiles16 - t_first;
    nvalid = nvalid < 0 ? 0 : (nvalid > NTW ? NTW : nvalid);
    WRsrc<NTW> R;
    R.w = make_rsrc(reinterpret_cast<const char*>(W) + (size_t)t_first * Gk * 1024,
                    (uint32_t)(nvalid * Gk * 1024));
    R.s = make_rsrc(Sp + (size_t)t_first * Gk * 16, (uint32_t)(nvalid * Gk * 32));
    if (MODE == W_ASYM)
      R.z = make_rsrc(reinterpret_cast<const char*>(Zp) + (size_t)t_first * Gk * 8,
                      (uint32_t)(nvalid * Gk * 8));
    else
      R.z = R.s;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const bool ok = t < nvalid;
      R.wo[t] = ok ? (uint32_t)(t * Gk * 1024 + lane * 16) : kOutOfRange;
      R.so[t] = ok ? (uint32_t)(t * Gk * 32 + (lane & 15) * 2) : kOutOfRange;
      R.zo[t] = ok ? (uint32_t)(t * Gk * 8) : kOutOfRange;
    }
    // zero-size resources: loads past the segment return zeros without a request,
    // which keeps the pipelined loop free of branches
    const rsrc_t rx0 = make_rsrc(X, 0);
    WRsrc<NTW> R0 = R;
    R0.w = make_rsrc(W, 0);
    R0.s = make_rsrc(Sp, 0);
    R0.z = R0.s;

#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = float4v{0.f, 0.f, 0.f, 0.f};

    const int nk = kb1 - kb0;
    WStage<NTW, MODE> S0, S1;
    u32x4 xr[MT];
    // prologue: block kb0 into LDS buffer 0 and registers S0; block kb0+1 in flight
    load_x<MT>(xr, rx, xoff, kb0);
    load_w(S0, R, kb0);
    __syncthreads();  // the previous segment's last reads of the LDS buffers are done
    store_x<MT>(lds, xr, tid);
    load_x<MT>(xr, nk > 1 ? rx : rx0, xoff, kb0 + 1);
    load_w(S1, nk > 1 ? R : R0, kb0 + 1);
    __syncthreads();

    // k-block i is in LDS buffer i%2 and in S(i%2); the activation registers hold
    // block i+1, the other weight stage block i+1 as well
    int i = 0;
    for (; i + 1 < nk; i += 2) {
      compute_kblock<MT, NTW, MODE>(lds, S0, acc, lane, magic);
      store_x<MT>(lds + XBUF, xr, tid);
      {
        const bool live = i + 2 < nk;
        load_x<MT>(xr, live ? rx : rx0, xoff, kb0 + i + 2);
        load_w(S0, live ? R : R0, kb0 + i + 2);
      }
      __syncthreads();
      compute_kblock<MT, NTW, MODE>(lds + XBUF, S1, acc, lane, magic);
      store_x<MT>(lds, xr, tid);
      {
        const bool live = i + 3 < nk;
        load_x<MT>(xr, live ? rx : rx0, xoff, kb0 + i + 3);
        load_w(S1, live ? R : R0, kb0 + i + 3);
      }
      __syncthreads();
    }
    if (i < nk) compute_kblock<MT, NTW, MODE>(lds, S0, acc, lane, magic);
  };

  // Y store of a finished tile: lane holds row 16i + lane%16 and the four columns
  // 16t + 4(lane/16) .. +3 of each of the wave's column tiles
  auto store_y = [&](int tt, const float4v (&acc)[MT][NTW]) {
    int tm, tn;
    tile_coords(tt, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    const int m0 = tm * BM;
    const int rows = a.M - m0 < BM ? a.M - m0 : BM;
    const rsrc_t ry = make_rsrc(Y + (size_t)m0 * a.N, (uint32_t)((size_t)rows * a.N * 2));
    const int t_first = tn * (BN / 16) + wave * NTW;
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if (t_first + t >= ntiles16) break;  // wave-uniform
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int r = 16 * i + (lane & 15);
        const uint32_t off = r < rows ? (uint32_t)(((size_t)r * a.N + (t_first + t) * 16 +
                                                    4 * (lane >> 4)) * 2)
                                      : kOutOfRange;
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = {pack_h2(acc[i][t][0], acc[i][t][1]), pack_h2(acc[i][t][2], acc[i][t][3])};
        __builtin_amdgcn_raw_buffer_store_b64(v, ry, off, 0u, 0);
      }
    }
  };

  float4v acc[MT][NTW];

  // ---- data-parallel rounds: tile it*grid + w, full K ----
  for (int it = 0; it < a.dp_rounds; ++it) {
    const int tt = it * a.grid + w;
    run_segment(tt, 0, Gk, acc);
    store_y(tt, acc);
  }
  if (a.sk_units == 0) return;

  // ---- stream-K stripe [u0, u1) over the remaining tiles' (tile, k-block) units ----
  const long u0 = (long)w * a.sk_per_wg;
  long u1 = u0 + a.sk_per_wg;
  if (u1 > a.sk_units) u1 = a.sk_units;
  for (long u = u0; u < u1;) {
    const int tl = (int)(u / Gk);  // tile index inside the stream-K part
    const int kb0 = (int)(u - (long)tl * Gk);
    const long rest = u1 - u;
    const int kb1 = rest < Gk - kb0 ? kb0 + (int)rest : Gk;
    const int tt = a.dp_rounds * a.grid + tl;
    run_segment(tt, kb0, kb1, acc);
    const bool first_seg = (u == u0);
    u += kb1 - kb0;
    if (kb0 == 0 && kb1 == Gk) {
      store_y(tt, acc);
      continue;
    }
    // partial tile: write this piece, count it, and finish the tile if last
    const int slot = 2 * w + (first_seg ? 0 : 1);
    {
      const rsrc_t rp = make_rsrc(part + (size_t)slot * PIECE, PIECE * 4);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, acc[i][t]), rp,
              (uint32_t)((((wave * MT + i) * NTW + t) * 64 + lane) * 16), 0u, kSC1);
    }
    const int w_first = (int)(((long)tl * Gk) / a.sk_per_wg);
    const int w_last = (int)(((long)(tl + 1) * Gk - 1) / a.sk_per_wg);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's sc1 stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __syncthreads();  // ... and so have every other thread's
    if (tid == 0)
      s_old = __hip_atomic_fetch_add(counters + tl, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int old = s_old;
    if (old != w_last - w_first) continue;
    // last arriver: sum the pieces in stripe order w_first .. w_last
    for (int wp = w_first; wp <= w_last; ++wp) {
      const int first_tile_of_wp = (int)(((long)wp * a.sk_per_wg) / Gk);
      const int sl = 2 * wp + (tl == first_tile_of_wp ? 0 : 1);
      const rsrc_t rp = make_rsrc(part + (size_t)sl * PIECE, PIECE * 4);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < NTW; ++t) {
          const float4v v = __builtin_bit_cast(
              float4v, __builtin_amdgcn_raw_buffer_load_b128(
                           rp, (uint32_t)((((wave * MT + i) * NTW + t) * 64 + lane) * 16), 0u,
                           kSC1));
          acc[i][t] = wp == w_first ? v : acc[i][t] + v;
        }
    }
    if (tid == 0)
      __hip_atomic_store(counters + tl, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    store_y(tt, acc);
  }
}

typedef void (*TiledFn)(const uint16_t*, const uint32_t*, const uint16_t*, const uint32_t*,
                        uint16_t*, float*, int*, TiledArgs);

struct TVariant {
  int MT, NTW;
  TiledFn sym, asym;
  const char* name;
};

#define W4A16_TILED(MT, NTW, NAME) \
  TVariant { MT, NTW, tiled_kernel<MT, NTW, W_SYM>, tiled_kernel<MT, NTW, W_ASYM>, NAME }

const TVariant kTiled[] = {
    W4A16_TILED(8, 4, "tiled_bm128_bn256"),
    W4A16_TILED(4, 4, "tiled_bm64_bn256"),
};
constexpr int kNumTiled = sizeof(kTiled) / sizeof(kTiled[0]);

}  // namespace

int tiled_variant_count() { return kNumTiled; }
const char* tiled_variant_name(int v) { return (v >= 0 && v < kNumTiled) ? kTiled[v].name : nullptr; }

int tiled_make_plan(int M, int N, int K, int mode, int variant, int grid, TiledPlan* p) {
  if (mode != W_SYM && mode != W_ASYM) return -8;
  if (variant < 0) variant = M > 64 ? 0 : 1;
  if (variant >= kNumTiled) return -8;
  const TVariant& v = kTiled[variant];
  const int BM = 16 * v.MT, BN = WAVES * 16 * v.NTW;
  const int Gk = K / KBLK;
  TiledPlan q;
  q.variant = variant;
  q.mode = mode;
  q.args.M = M;
  q.args.N = N;
  q.args.K = K;
  q.args.tiles_m = (M + BM - 1) / BM;
  q.args.tiles_n = (N + BN - 1) / BN;
  q.args.group_m = 8;
  const long T = (long)q.args.tiles_m * q.args.tiles_n;
  if (T > (1L << 30)) return -2;
  if (grid <= 0) {
    // one workgroup per compute unit; fewer for small problems, so that a stripe
    // holds at least a few k-blocks
    const long min_units = 8;
    long g = (T * Gk + min_units - 1) / min_units;
    grid = (int)(g < 256 ? (g < 1 ? 1 : g) : 256);
  }
  q.args.grid = grid;
  const long full = T / grid;
  long dp_tiles;
  if (T % grid == 0) dp_tiles = T;
  else if (full >= 1) dp_tiles = (full - 1) * grid;
  else dp_tiles = 0;
  q.args.dp_rounds = (int)(dp_tiles / grid);
  const long sk_tiles = T - dp_tiles;
  q.args.sk_units = (long long)sk_tiles * Gk;
  q.args.sk_per_wg = (q.args.sk_units + grid - 1) / grid;
  if (q.args.sk_per_wg < 1) q.args.sk_per_wg = 1;
  q.counters = (int)sk_tiles;
  q.part_floats = sk_tiles ? (size_t)2 * grid * BM * BN : 0;
  q.wgs = grid;
  q.threads = 64 * WAVES;
  *p = q;
  return 0;
}

hipError_t tiled_launch(const TiledPlan& p, const uint16_t* X, const void* w, const uint16_t* sp,
                        const uint32_t* zp, uint16_t* Y, float* part, int* counters,
                        hipStream_t st) {
  const TVariant& v = kTiled[p.variant];
  TiledFn fn = p.mode == W_ASYM ? v.asym : v.sym;
  hipLaunchKernelGGL(fn, dim3(p.wgs), dim3(p.threads), 0, st, X,
                     reinterpret_cast<const uint32_t*>(w), sp, zp, Y, part, counters, p.args);
  return hipGetLastError();
}

}  // namespace w4a16
