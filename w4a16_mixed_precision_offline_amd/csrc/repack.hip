// Offline repack of group-quantized INT4 weights into the MFMA-fragment layout,
// its exact inverse, and the unfused baseline's dequantization.
//
// The pages describe a one-time, load-time reshuffle of weights and scales into
// a tiled layout that suits the matrix instructions ("Marlin / GPTQ-Marlin",
// brain.gartu.xyz, section "2. Tiled layout et repacking"; "Marlin Project
// Overview", vecbase.com, "Key Techniques": reshuffling for access patterns).
// The layout itself is this library's own (described in internal.h): each
// repacked word is one canonical word with its nibbles permuted, so the repack
// is a gather plus an in-register nibble shuffle, reading and writing every
// byte exactly once.
#include "internal.h"

namespace w4a16 {

namespace {

// canonical word (rows 8i+e at nibble e) -> repacked word (row e at nib_pos(e))
__device__ __forceinline__ uint32_t shuffle_to_repacked(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) r |= ((v >> (4 * e)) & 15u) << (4 * nib_pos(e));
  return r;
}
__device__ __forceinline__ uint32_t shuffle_to_canonical(uint32_t v) {
  uint32_t r = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) r |= ((v >> (4 * nib_pos(e))) & 15u) << (4 * e);
  return r;
}

// Repacked word index o -> canonical word index (row i of q[K/8][N], column n).
__device__ __forceinline__ void repacked_to_canonical(long o, int Gk, int N, long* ci) {
  const int j = (int)(o & 3);
  const int l = (int)((o >> 2) & 63);
  const long b = o >> 8;
  const long t = b / Gk;
  const int kb = (int)(b - t * Gk);
  const long i = 16L * kb + 4 * j + (l >> 4);
  const long n = 16L * t + (l & 15);
  *ci = i * N + n;
}

template <bool TO_REPACKED>
__global__ void codes_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                             long total, int Gk, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    long ci;
    repacked_to_canonical(o, Gk, N, &ci);
    if (TO_REPACKED) dst[o] = shuffle_to_repacked(src[ci]);
    else dst[ci] = shuffle_to_canonical(src[o]);
  }
}

// Canonical group row of half h of 128-row block kb: SH = 2 for groups of 64 rows,
// otherwise gpb = group / 128 blocks per group.
__device__ __forceinline__ long group_row(int kb, int h, int SH, int gpb) {
  return SH == 2 ? 2L * kb + h : (long)(kb / gpb);
}

// scales: repacked index o = ((t*Gk + kb)*16 + c)*SH + h  <->  canonical s[row][16t + c]
// (a group spanning gpb blocks is stored gpb times, and the inverse reads the first copy)
template <bool TO_REPACKED>
__global__ void scales_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                              long total, int Gk, int gpb, int SH, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int h = SH == 2 ? (int)(o & 1) : 0;
    const long oc = SH == 2 ? o >> 1 : o;
    const int c = (int)(oc & 15);
    const long tk = oc >> 4;
    const long t = tk / Gk;
    const int kb = (int)(tk - t * Gk);
    const long ci = group_row(kb, h, SH, gpb) * N + 16 * t + c;
    if (TO_REPACKED) dst[o] = src[ci];
    else if (SH == 2 || kb % gpb == 0) dst[ci] = src[o];
  }
}

// zero-points: repacked word o = ((t*Gk + kb)*SH + h)*2 + w  <->  canonical word
// [row][2t + w]
template <bool TO_REPACKED>
__global__ void zeros_kernel(const uint32_t* __restrict__ src, uint32_t* __restrict__ dst,
                             long total, int Gk, int gpb, int SH, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int w = (int)(o & 1);
    const long oh = o >> 1;
    const int h = SH == 2 ? (int)(oh & 1) : 0;
    const long tk = SH == 2 ? oh >> 1 : oh;
    const long t = tk / Gk;
    const int kb = (int)(tk - t * Gk);
    const long ci = group_row(kb, h, SH, gpb) * (N / 8) + 2 * t + w;
    if (TO_REPACKED) dst[o] = src[ci];
    else if (SH == 2 || kb % gpb == 0) dst[ci] = src[o];
  }
}

// Unfused baseline dequantization: Wt[n][k] = RNE((q[k][n] - z[k/g][n]) * s[k/g][n]).
// (q - z) * s is exact in fp32 (a 5-bit integer times an 11-bit significand), so the
// single conversion to fp16 rounds the exact value to nearest-even.
// A workgroup transposes a tile of 32 canonical word rows (256 K) x 64 columns through
// LDS: the words are read along N (256 contiguous bytes per row) and the fp16 rows of Wt
// are written along K (512 contiguous bytes per column), so both sides coalesce.
constexpr int DQ_ROWS = 32, DQ_COLS = 64;
constexpr int DQ_STRIDE = DQ_ROWS * 16 + 16;  // LDS bytes per column (+16 against conflicts)
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ q,
                                                      const uint16_t* __restrict__ s,
                                                      const uint32_t* __restrict__ z,
                                                      uint16_t* __restrict__ Wt, int K, int N,
                                                      int group) {
  __shared__ __attribute__((aligned(16))) char tile[DQ_COLS * DQ_STRIDE];
  const int t = threadIdx.x;
  const int n0 = blockIdx.x * DQ_COLS;
  const long i0 = (long)blockIdx.y * DQ_ROWS;
  const long rows = K / 8;
  // read and dequantize: thread t takes column n0 + t%64 of rows i0 + t/64 + 4r
  {
    const int c = t & 63;
    const int n = n0 + c;
#pragma unroll
    for (int r = 0; r < DQ_ROWS / 4; ++r) {
      const int il = (t >> 6) + 4 * r;
      const long i = i0 + il;
      if (n >= N || i >= rows) continue;
      const int g = (int)((8 * i) / group);
      const uint32_t v = q[i * N + n];
      const float sc = (float)__builtin_bit_cast(_Float16, s[(long)g * N + n]);
      int zz = 8;
      if (z) zz = (int)((z[(long)g * (N / 8) + n / 8] >> (4 * (n & 7))) & 15u);
      uint16_t out[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int qq = (int)((v >> (4 * e)) & 15u);
        out[e] = __builtin_bit_cast(uint16_t, (_Float16)((float)(qq - zz) * sc));
      }
      uint4 pk;
      pk.x = out[0] | ((uint32_t)out[1] << 16);
      pk.y = out[2] | ((uint32_t)out[3] << 16);
      pk.z = out[4] | ((uint32_t)out[5] << 16);
      pk.w = out[6] | ((uint32_t)out[7] << 16);
      *reinterpret_cast<uint4*>(tile + c * DQ_STRIDE + il * 16) = pk;
    }
  }
  __syncthreads();
  // write: element e = t + 256r of the tile is column e / 32, word row e % 32
#pragma unroll
  for (int r = 0; r < DQ_ROWS * DQ_COLS / 256; ++r) {
    const int e = t + 256 * r;
    const int c = e / DQ_ROWS, il = e % DQ_ROWS;
    const int n = n0 + c;
    const long i = i0 + il;
    if (n >= N || i >= rows) continue;
    *reinterpret_cast<uint4*>(Wt + (long)n * K + 8 * i) =
        *reinterpret_cast<const uint4*>(tile + c * DQ_STRIDE + il * 16);
  }
}

// ---- 2:4 sparse compress / decompress (symmetric codes, zero code 8) ----------------
// Layout (own design, follows the operand semantics of v_smfmac_f32_16x16x64_f16,
// measured on MI355X): per (tile t, 128-row block kb), lane l owns column
// n = 16t + l%16 and, for each half h (0, 1) of the block, the 16 dense rows
// kb*128 + 64h + 16(l/16) + [0, 16), i.e. four aligned runs of 4.  From run g it keeps
// two codes (the non-zero ones, topped up with the lowest free positions), in
// ascending position, as elements 2g and 2g+1 of a word (nibble order as the dense
// layout: element e at nibble e/2 + 4(e%2)), and writes the positions as 2-bit fields
// at bits 16h + 2e of one metadata word per lane and block.
//   vp  : [N/16][K/128][64 lanes][2 words]   idx : [N/16][K/128][64 lanes] words
__global__ void sparse_compress_kernel(const uint32_t* __restrict__ q, uint32_t* __restrict__ vp,
                                       uint32_t* __restrict__ meta, int* __restrict__ bad,
                                       long total, int Gk, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int l = (int)(o & 63);
    const long b = o >> 6;
    const long t = b / Gk;
    const int kb = (int)(b - t * Gk);
    const long n = 16 * t + (l & 15);
    uint32_t mw = 0;
    int nbad = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // canonical words holding rows kb*128 + 64h + 16(l/16) + 0..7 and 8..15
      const long i0 = (long)kb * 16 + 8 * h + 2 * (l >> 4);
      const uint64_t codes = (uint64_t)q[i0 * N + n] | ((uint64_t)q[(i0 + 1) * N + n] << 32);
      uint32_t word = 0;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        int keep[2] = {0, 0}, nk = 0;
        for (int p = 0; p < 4; ++p) {
          const uint32_t c = (uint32_t)(codes >> (4 * (4 * g + p))) & 15u;
          if (c != 8u) {
            if (nk < 2) keep[nk] = p;
            ++nk;
          }
        }
        if (nk > 2) ++nbad;
        // top up with the lowest positions not already kept (ascending order kept)
        for (int p = 0; nk < 2 && p < 4; ++p) {
          if (nk == 1 && keep[0] == p) continue;
          if (nk == 1 && p < keep[0]) { keep[1] = keep[0]; keep[0] = p; }
          else keep[nk] = p;
          ++nk;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int e = 2 * g + u;
          const uint32_t c = (uint32_t)(codes >> (4 * (4 * g + keep[u]))) & 15u;
          word |= c << (4 * nib_pos(e));
          mw |= (uint32_t)keep[u] << (16 * h + 2 * e);
        }
      }
      vp[o * 2 + h] = word;
    }
    meta[o] = mw;
    if (nbad) atomicAdd(bad, nbad);
  }
}

__global__ void sparse_decompress_kernel(const uint32_t* __restrict__ vp,
                                         const uint32_t* __restrict__ meta,
                                         uint32_t* __restrict__ q, long total, int Gk, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int l = (int)(o & 63);
    const long b = o >> 6;
    const long t = b / Gk;
    const int kb = (int)(b - t * Gk);
    const long n = 16 * t + (l & 15);
    const uint32_t mw = meta[o];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = vp[o * 2 + h];
      uint64_t codes = 0x8888888888888888ull;  // every position zero (code 8) ...
#pragma unroll
      for (int e = 0; e < 8; ++e) {             // ... except the kept ones
        const int g = e >> 1;
        const int p = (int)((mw >> (16 * h + 2 * e)) & 3u);
        const uint64_t c = (word >> (4 * nib_pos(e))) & 15u;
        const int sh = 4 * (4 * g + p);
        codes = (codes & ~(15ull << sh)) | (c << sh);
      }
      const long i0 = (long)kb * 16 + 8 * h + 2 * (l >> 4);
      q[i0 * N + n] = (uint32_t)codes;
      q[(i0 + 1) * N + n] = (uint32_t)(codes >> 32);
    }
  }
}

__global__ void zero_int_kernel(int* p) { *p = 0; }

// The whole repack in one launch.  Workgroups [0, nA) repack codes: workgroup
// kb * pairs + p takes the 16-column tiles 2p and 2p + 1 of the 128-row block kb, so that
// for each word j its 128 threads read 4 canonical rows x 32 columns, i.e. whole 128-byte
// lines, and consecutive workgroups read neighbouring lines of the same rows.  Thread
// (h = tile of the pair, lane l) writes lane l's 16 bytes of its block: words j = 0..3
// hold rows 16kb + 4j + l/16 of column 32p + 16h + l%16.  The workgroups after nA copy the
// scales, then the zero-points, one element per thread (layouts as in scales_kernel and
// zeros_kernel).
__global__ __launch_bounds__(128) void repack_all_kernel(
    const uint32_t* __restrict__ q, uint32_t* __restrict__ wp, const uint16_t* __restrict__ s,
    uint16_t* __restrict__ sp, const uint32_t* __restrict__ z, uint32_t* __restrict__ zp, int Gk,
    int N, int gpb, int SH, long nA, long nS, long stot, long ztot) {
  const long b = blockIdx.x;
  const int tid = threadIdx.x;
  if (b < nA) {
    const int tiles = N / 16;
    const long pairs = (tiles + 1) / 2;
    const long kb = b / pairs;
    const long p = b - kb * pairs;
    const int h = tid >> 6, l = tid & 63;
    const long t = 2 * p + h;
    if (t >= tiles) return;  // odd tile count: the last pair has one tile
    const long n = 16 * t + (l & 15);
    uint4 v;
    uint32_t* vw = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long i = 16 * kb + 4 * j + (l >> 4);
      vw[j] = shuffle_to_repacked(q[i * N + n]);
    }
    *reinterpret_cast<uint4*>(wp + (t * Gk + kb) * 256 + 4 * l) = v;
    return;
  }
  if (b < nA + nS) {
    const long o = (b - nA) * 128 + tid;
    if (o >= stot) return;
    const int hh = SH == 2 ? (int)(o & 1) : 0;
    const long oc = SH == 2 ? o >> 1 : o;
    const int c = (int)(oc & 15);
    const long tk = oc >> 4;
    const long tt = tk / Gk;
    const int kb = (int)(tk - tt * Gk);
    sp[o] = s[group_row(kb, hh, SH, gpb) * N + 16 * tt + c];
    return;
  }
  const long o = (b - nA - nS) * 128 + tid;
  if (o >= ztot) return;
  const int w = (int)(o & 1);
  const long oh = o >> 1;
  const int hh = SH == 2 ? (int)(oh & 1) : 0;
  const long tk = SH == 2 ? oh >> 1 : oh;
  const long tt = tk / Gk;
  const int kb = (int)(tk - tt * Gk);
  zp[o] = z[group_row(kb, hh, SH, gpb) * (N / 8) + 2 * tt + w];
}

inline int grid_for(long total, int threads) {
  long b = (total + threads - 1) / threads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_repack(const int32_t* q, const uint16_t* s, const int32_t* z, uint32_t* wp,
                         uint16_t* sp, uint32_t* zp, int K, int N, int group, hipStream_t st) {
  const int Gk = K / KBLK, SH = group == 64 ? 2 : 1, gpb = SH == 2 ? 1 : group / KBLK;
  const long stot = (long)Gk * N * SH, ztot = z ? (long)Gk * N / 8 * SH : 0;
  const long nA = (long)((N / 16 + 1) / 2) * Gk, nS = (stot + 127) / 128, nZ = (ztot + 127) / 128;
  repack_all_kernel<<<(unsigned)(nA + nS + nZ), 128, 0, st>>>(
      reinterpret_cast<const uint32_t*>(q), wp, s, sp, reinterpret_cast<const uint32_t*>(z), zp,
      Gk, N, gpb, SH, nA, nS, stot, ztot);
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t* wp, const uint16_t* sp, const uint32_t* zp, int32_t* q,
                         uint16_t* s, int32_t* z, int K, int N, int group, hipStream_t st) {
  const int Gk = K / KBLK, SH = group == 64 ? 2 : 1, gpb = SH == 2 ? 1 : group / KBLK;
  const long wtot = (long)K * N / 8, stot = (long)Gk * N * SH, ztot = (long)Gk * N / 8 * SH;
  codes_kernel<false><<<grid_for(wtot, 256), 256, 0, st>>>(
      wp, reinterpret_cast<uint32_t*>(q), wtot, Gk, N);
  scales_kernel<false><<<grid_for(stot, 256), 256, 0, st>>>(sp, s, stot, Gk, gpb, SH, N);
  if (zp) zeros_kernel<false><<<grid_for(ztot, 256), 256, 0, st>>>(
      zp, reinterpret_cast<uint32_t*>(z), ztot, Gk, gpb, SH, N);
  return hipGetLastError();
}

hipError_t launch_sparse_compress(const int32_t* q, const uint16_t* s, uint32_t* vp,
                                  uint32_t* meta, uint16_t* sp, int* bad, int K, int N, int group,
                                  hipStream_t st) {
  const int Gk = K / KBLK, gpb = group / KBLK;
  const long tot = (long)(N / 16) * Gk * 64, stot = (long)Gk * N;
  zero_int_kernel<<<1, 1, 0, st>>>(bad);
  sparse_compress_kernel<<<grid_for(tot, 256), 256, 0, st>>>(
      reinterpret_cast<const uint32_t*>(q), vp, meta, bad, tot, Gk, N);
  scales_kernel<true><<<grid_for(stot, 256), 256, 0, st>>>(s, sp, stot, Gk, gpb, 1, N);
  return hipGetLastError();
}

hipError_t launch_sparse_decompress(const uint32_t* vp, const uint32_t* meta, const uint16_t* sp,
                                    int32_t* q, uint16_t* s, int K, int N, int group,
                                    hipStream_t st) {
  const int Gk = K / KBLK, gpb = group / KBLK;
  const long tot = (long)(N / 16) * Gk * 64, stot = (long)Gk * N;
  sparse_decompress_kernel<<<grid_for(tot, 256), 256, 0, st>>>(
      vp, meta, reinterpret_cast<uint32_t*>(q), tot, Gk, N);
  scales_kernel<false><<<grid_for(stot, 256), 256, 0, st>>>(sp, s, stot, Gk, gpb, 1, N);
  return hipGetLastError();
}

namespace {

// MXFP4 (OCP Microscaling FP4: E2M1 codes, one E8M0 scale per 32 rows along K), for
// the block-scaled matrix instruction, which takes the micro-block scales itself (the
// pages' FP4-with-micro-block-scales design, dingiv.github.io "Marlin", section "与
// Blackwell NVFP4 的对比").  Code word o = ((t*Gk + kb)*64 + l)*4 + w of the repacked
// array is canonical word kb*16 + 4(l/16) + w of column 16t + l%16, unchanged: its
// nibbles already hold rows 8w .. 8w+7 of lane l's 32 rows, low nibble first, which is
// the operand order of the instruction.  Scale byte ((t*Gk + kb)*64 + l) is
// e[kb*4 + l/16][16t + l%16]; each thread writes the 4 bytes of lanes 4j .. 4j+3.
__global__ void mx_codes_kernel(const uint32_t* __restrict__ q, uint32_t* __restrict__ wp,
                                long total, int Gk, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int w = (int)(o & 3), l = (int)((o >> 2) & 63);
    const long blk = o >> 8;  // t*Gk + kb
    const long t = blk / Gk, kb = blk - t * Gk;
    wp[o] = q[(kb * 16 + 4 * (l >> 4) + w) * (long)N + 16 * t + (l & 15)];
  }
}
__global__ void mx_scales_kernel(const uint8_t* __restrict__ e, uint32_t* __restrict__ sp,
                                 long total, int Gk, int N) {
  for (long o = blockIdx.x * (long)blockDim.x + threadIdx.x; o < total;
       o += (long)gridDim.x * blockDim.x) {
    const int j = (int)(o & 15);
    const long blk = o >> 4;
    const long t = blk / Gk, kb = blk - t * Gk;
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int l = 4 * j + b;
      v |= (uint32_t)e[(kb * 4 + (l >> 4)) * (long)N + 16 * t + (l & 15)] << (8 * b);
    }
    sp[o] = v;
  }
}

}  // namespace

hipError_t launch_mx_repack(const int32_t* q, const uint8_t* e, uint32_t* wp, uint8_t* sp,
                            int K, int N, hipStream_t st) {
  const int Gk = K / KBLK;
  const long wtot = (long)K * N / 8, stot = (long)K * N / 128;
  mx_codes_kernel<<<grid_for(wtot, 256), 256, 0, st>>>(reinterpret_cast<const uint32_t*>(q), wp,
                                                       wtot, Gk, N);
  mx_scales_kernel<<<grid_for(stot, 256), 256, 0, st>>>(e, reinterpret_cast<uint32_t*>(sp), stot,
                                                        Gk, N);
  return hipGetLastError();
}

hipError_t launch_dequant(const int32_t* q, const uint16_t* s, const int32_t* z, uint16_t* Wt,
                          int K, int N, int group, hipStream_t st) {
  const dim3 grid((unsigned)((N + DQ_COLS - 1) / DQ_COLS),
                  (unsigned)((K / 8 + DQ_ROWS - 1) / DQ_ROWS));
  dequant_kernel<<<grid, 256, 0, st>>>(reinterpret_cast<const uint32_t*>(q), s,
                                       reinterpret_cast<const uint32_t*>(z), Wt, K, N, group);
  return hipGetLastError();
}

}  // namespace w4a16
