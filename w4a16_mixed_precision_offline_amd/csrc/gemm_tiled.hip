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
//   * Per 128-row k-block the activation tile (BM x 128 fp16) and each wave's
//     weight blocks, scales (and zero-points) are loaded straight into LDS
//     (direct-to-LDS buffer loads) into a ring of NS stages; loads for k-block
//     kb + NS - 1 are issued, one per matrix-instruction group, while kb is
//     computed.  The activation tile is XOR-swizzled by 16-byte chunk so that a
//     fragment read (lane l: row 16i + l%16, 8 halves at 32j + 8(l/16)) hits every
//     LDS bank once.
//   * A wave's weight block is 1 KiB in the repacked layout: lane l's 16 bytes are
//     already the operand fragment of the four v_mfma_f32_16x16x32_f16 of the
//     block.  Codes become exact fp16 (q - z) with the 0x6400 exponent trick and
//     are multiplied by the fp16 scale (one rounding of W, as in the dequantized
//     fp16 weight), so the accumulators need no per-block rescaling.
//   * W is the MFMA's A operand and X its B operand: a lane's accumulator then
//     holds four consecutive columns of one row of Y (one 8-byte store).
//   * Work split: the first full rounds of tiles are handed out data-parallel (one
//     tile per workgroup per round, full K); the remaining tiles' (tile, k-block)
//     units are cut into equal contiguous stripes over all workgroups (stream-K).
//     A workgroup stores the fp32 partial tile of its first and last stripe
//     segment when the segment does not cover the whole K range; a second kernel
//     sums each cut tile's pieces in stripe order (a fixed order, hence bitwise
//     reproducible results) and writes Y.
//   * The same skeleton runs the 2:4 format (kept codes and positions in LDS,
//     v_smfmac_f32_16x16x64_f16) and the fp16 baseline (fp16 weight fragments,
//     no unpacking).
#include "internal.h"

namespace w4a16 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
// cache-policy bits of buffer instructions on gfx950

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}

// Direct-to-LDS loads.  The 128-bit buffer descriptor is built by hand (raw
// buffer, stride 0, num_records = bytes) so that it can be handed to inline asm;
// lane L of a 16-byte (4-byte) load writes LDS bytes [16L, 16L+16) ([4L, 4L+4))
// after the base held in M0, and lanes out of range write zeros.  The loads are
// issued from inline asm because the compiler, unable to tell the destination
// stage from the stage being read, would otherwise wait for every just-issued
// load before the next LDS read and serialize loading with computing; their
// completion is ordered explicitly (s_waitcnt vmcnt + s_barrier) by the caller.
// Writing M0 needs one wait state before the load that uses it.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}
__device__ __forceinline__ void dma16(u32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
#else
  (void)r, (void)lds, (void)voff, (void)soff;  // host pass: device-only instruction
#endif
}
__device__ __forceinline__ void dma4(u32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
#else
  (void)r, (void)lds, (void)voff, (void)soff;  // host pass: device-only instruction
#endif
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

constexpr int WAVES = 4;

typedef short short2v __attribute__((ext_vector_type(2)));
typedef int int8v __attribute__((ext_vector_type(8)));

// fp8 activations: 8 codes of one repacked word -> the 8 OCP E4M3 bytes of the exact
// integers q - z (rows 0..7 in bytes 0..7): exact q - z in fp16 by the 0x6400 trick, then
// a unit-scale conversion per pair (every integer in [-15, 15] is exact in E4M3).
__device__ __forceinline__ uint2 dequant_fp8(uint32_t w, half2v c0, half2v c1, uint32_t magic) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const half2v h0 = __builtin_bit_cast(half2v, and_or(w, 0x000F000Fu, magic)) + c0;
  const half2v h1 =
      __builtin_elementwise_fma(__builtin_bit_cast(half2v, and_or(w, 0x00F000F0u, magic)), sixteenth, c1);
  const half2v h2 = __builtin_bit_cast(half2v, and_or(w8, 0x000F000Fu, magic)) + c0;
  const half2v h3 =
      __builtin_elementwise_fma(__builtin_bit_cast(half2v, and_or(w8, 0x00F000F0u, magic)), sixteenth, c1);
  short2v lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(lo, h0, 1.0f, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(lo, h1, 1.0f, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(hi, h2, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(hi, h3, 1.0f, true);
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// Per-wave weight sources of the current tile: resources over the wave's valid
// column tiles, per-lane offsets of the column-tile part of each address
// (kOutOfRange for tiles past N and for idle lanes: they read zeros), the
// k-block part goes to the scalar offset.
template <int NTW>
struct WSrc {
  u32x4 w, s, z;
  uint32_t wo[NTW];  // codes: tile t, 16 bytes of lane L
  uint32_t so;       // scales: lane L < 8*NTW loads the scale pair 2(L%8), +1 of tile L/8
  uint32_t zo;       // zero-points: lane L < 2*NTW loads half L%2 of tile L/2's 64-bit word
};

// LDS of one pipeline stage, per wave: NTW 1 KiB code blocks, then 256 bytes of
// scales (tile t, column c at 32t + 2c; with groups of 64 rows, half h at
// 64t + 4c + 2h; the DMA writes 4 bytes per lane, so the slot spans all 64 lanes) and
// 256 bytes of zero-points (tile t at 8t; with groups of 64, half h at 16t + 8h).
template <int NTW, int MODE>
struct WLds {
  // dense: NTW 1 KiB code blocks.  2:4: NTW 512-byte blocks of kept codes (lane l's
  // two words at 8l), then NTW 256-byte blocks of positions (lane l's word at 4l).
  static constexpr bool SP = MODE == W_SP24;
  static constexpr int META = NTW * 512;
  // fp16 weights (baseline): per column tile four 1 KiB fragments (k-steps 0..3)
  static constexpr int CODES = SP ? NTW * 768 : MODE == W_FP16 ? NTW * 4096 : NTW * 1024;
  static constexpr int SCALES = CODES;
  static constexpr int ZEROS = CODES + 256;
  static constexpr int BYTES = CODES + 512;
};


// Activation tile in LDS: BM rows of 256 bytes (one 128-row k-block of X), no
// padding; the 16-byte chunk c of row r sits at chunk position c ^ (r % 16), so
// that the 16 lanes of a fragment read (16 rows, one chunk) hit 16 different
// chunk positions, i.e. all 64 banks once.
__device__ __forceinline__ uint32_t swz(int r, int c) { return (uint32_t)(r * 256 + ((c ^ (r & 15)) << 4)); }

// fp8 activations: BM rows of 128 bytes; chunk c of row r at chunk position c ^ ((r >> 1) & 7).
// A fragment read (lane l: row 16i + l%16, the 8 bytes at 32j + 8(l/16)) then puts the 16
// rows of one lane group on 16 different (row parity, chunk position) pairs and the 4
// groups on different dwords of them: every bank is read exactly twice per instruction.
__device__ __forceinline__ uint32_t swz8(int r, int c) {
  return (uint32_t)(r * 128 + ((c ^ ((r >> 1) & 7)) << 4));
}

// Direct-to-LDS loads of one k-block of X: each wave instruction writes 1 KiB of
// LDS (lane L -> bytes 16L..16L+15 after the destination base), i.e. 4 rows; lane L
// of instruction c therefore fetches row 4(wave*MT + c) + L/16 and the global chunk
// that belongs at chunk position L%16.  Rows past M read zeros (out of range).

// The direct-to-LDS loads of one k-block for one wave, as a list of NV single
// instructions (MT activation quarters-of-rows blocks, NTW code blocks, the
// scales and, for zero-points, one more) so that they can be spread over the
// matrix work of the preceding k-block instead of being issued in one burst
// (a burst of 4 waves x NV loads fills the address queue of the CU and stalls
// the waves before their MFMAs start).
template <int MT, int NTW, int MODE, int NWV = WAVES>
struct DmaPlan {
  // activation loads per wave: 1 KiB each, 4 rows of fp16 or 8 rows of fp8; the NWV waves
  // share the BM-row tile
  static constexpr int NX = (mode_fp8(MODE) ? MT / 2 : MT) * WAVES / NWV;
  static_assert(NX >= 1, "every wave loads part of the activation tile");
  static constexpr uint32_t XKB = mode_fp8(MODE) ? 128u : 256u;  // X bytes per row and k-block
  // 2:4: two tiles' kept codes per 16-byte load, all four tiles' positions in one
  static constexpr int NW = MODE == W_SP24 ? NTW / 2 + NTW / 4 : MODE == W_FP16 ? 4 * NTW : NTW;
  static constexpr int NV = NX + NW + (mode_asym(MODE) ? 2 : MODE == W_FP16 ? 0 : 1);
  static constexpr uint32_t SH = mode_scale64(MODE) ? 2u : 1u;  // 32-byte scale rows per block
  u32x4 rx;
  uint32_t xoff[NX];
  WSrc<NTW> R;
  uint32_t xdst, wdst;  // LDS addresses: activation stage, this wave's weight slot
  int wave, kb;
  __device__ __forceinline__ void issue(int q) const {
    typedef WLds<NTW, MODE> L;
    if (q < NX) {
      dma16(rx, xdst + (wave * NX + q) * 1024, xoff[q], (uint32_t)kb * XKB);
    } else if (MODE == W_SP24 && q < NX + NTW / 2) {
      const int c = q - NX;  // kept codes of tiles 2c, 2c+1
      dma16(R.w, wdst + c * 1024, R.wo[c], (uint32_t)kb * 512u);
    } else if (MODE == W_SP24 && q < NX + NW) {
      dma16(R.z, wdst + L::META + (q - NX - NTW / 2) * 1024, R.zo, (uint32_t)kb * 256u);
    } else if (MODE == W_FP16 && q < NX + NW) {
      const int t = (q - NX) >> 2, j = (q - NX) & 3;  // rows 32j.. of column tile t
      dma16(R.w, wdst + (t * 4 + j) * 1024, R.wo[t], (uint32_t)kb * 256u + 64u * j);
    } else if (mode_dense4(MODE) && q < NX + NTW) {
      const int t = q - NX;
      dma16(R.w, wdst + t * 1024, R.wo[t], (uint32_t)kb * 1024u);
    } else if (MODE != W_FP16 && q == NX + NW) {
      dma4(R.s, wdst + L::SCALES, R.so, (uint32_t)kb * 32u * SH);
    } else if (mode_asym(MODE) && q == NX + NW + 1) {
      dma4(R.z, wdst + L::ZEROS, R.zo, (uint32_t)kb * 8u * SH);
    }
  }
};

// One k-block: the wave's weight codes, scales (and zero-points) come from its
// LDS slot, the activation fragments from the shared tile; 4 k-steps of 32.
// Software pipeline, one group per (k-step j, row tile i): the group issues the
// LDS read of the fragment three groups ahead, unpacks its share of the column tiles
// of step j+1 (tiles t = i, i + MT, ...), and runs the NTW MFMAs of (j, i).  Scheduling barriers between the groups
// keep that order, so LDS latency hides behind the matrix work.
template <int MT, int NTW, int MODE, class DP>
__device__ __forceinline__ void compute_kblock(const char* xb, const char* wl,
                                               float4v (&acc)[MT][NTW], const uint32_t (&aoff)[4],
                                               int lane, uint32_t magic,
                                               const DP& dma) {
  constexpr int NVL = DP::NV;
  constexpr int G = 4 * MT;  // groups per k-block
  u32x4 wv[NTW];
  half2v c0[NTW], c1[NTW], s2[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) wv[t] = *reinterpret_cast<const u32x4*>(wl + t * 1024 + lane * 16);
  // scale and zero-point offsets of half h of the block for every column tile (with
  // groups of 64 rows the second half's values replace the first's once step 1 has
  // been unpacked: steps 0, 1 are rows 0-63, steps 2, 3 rows 64-127)
  auto load_consts = [&](int h) {
    constexpr bool G64 = mode_g64(MODE);
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const int c = lane & 15;
      const _Float16 sc = *reinterpret_cast<const _Float16*>(
          wl + WLds<NTW, MODE>::SCALES + (G64 ? t * 64 + c * 4 + h * 2 : t * 32 + c * 2));
      s2[t] = half2v{sc, sc};
      int zq = 8;
      if (mode_asym(MODE)) {
        const uint32_t zw = *reinterpret_cast<const uint32_t*>(
            wl + WLds<NTW, MODE>::ZEROS + (G64 ? t * 16 + h * 8 : t * 8) + (c >> 3) * 4);
        zq = (int)((zw >> (4 * (c & 7))) & 15u);
      }
      const _Float16 a0 = (_Float16)(float)(-1024 - zq);
      const _Float16 a1 = (_Float16)(float)(-64 - zq);
      c0[t] = half2v{a0, a0};
      c1[t] = half2v{a1, a1};
    }
  };
  load_consts(0);
  // fragment ring: group g's activation fragment is read PF groups ahead
  constexpr int PF = 3;
  half8 ar[PF + 1];
#pragma unroll
  for (int g = 0; g < PF; ++g)
    if (g < G) ar[g] = *reinterpret_cast<const half8*>(xb + aoff[g / MT] + (g % MT) * 4096);
  half8 b[2][NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) b[0][t] = dequant_scaled(wv[t][0], c0[t], c1[t], s2[t], magic);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int g = j * MT + i;
      // loads of a later k-block: q = g, g + G, ... (one per group when NV <= G)
#pragma unroll
      for (int q = g; q < NVL; q += G) dma.issue(q);
      if (g + PF < G) {
        const int gj = (g + PF) / MT, gi = (g + PF) % MT;
        ar[(g + PF) % (PF + 1)] = *reinterpret_cast<const half8*>(xb + aoff[gj] + gi * 4096);
      }
      if (mode_g64(MODE) && j == 1 && i == 0) load_consts(1);
      // unpack the column tiles t = i, i + MT, ... of step j + 1
      if (j < 3) {
#pragma unroll
        for (int t = i; t < NTW; t += MT)
          b[(j + 1) & 1][t] = dequant_scaled(wv[t][j + 1], c0[t], c1[t], s2[t], magic);
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j & 1][t], ar[g % (PF + 1)],
                                                          acc[i][t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One k-block of the 2:4 format: per column tile, lane l holds two words of kept
// codes (half h = 0, 1 of the block's 64-row halves; column l%16) and one word of
// positions (two 16-bit sets, selected by the instruction's abid).  Each group
// (half h, row tile i) reads the two 32-row activation fragments 2h and 2h+1 of
// row tile i and runs v_smfmac_f32_16x16x64_f16 with the unpacked weights as the
// sparse operand: half the matrix instructions and half the unpacking of the dense
// format for the same k-block.
template <int MT, int NTW, class DP>
__device__ __forceinline__ void compute_kblock_sp24(const char* xb, const char* wl,
                                                    float4v (&acc)[MT][NTW],
                                                    const uint32_t (&aoff)[4], int lane,
                                                    uint32_t magic,
                                                    const DP& dma) {
  typedef WLds<NTW, W_SP24> L;
  constexpr int G = 2 * MT;  // groups per k-block
  constexpr int NVL = DP::NV;
  uint2 wv[NTW];
  int meta[NTW];
  half2v s2[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    wv[t] = *reinterpret_cast<const uint2*>(wl + t * 512 + lane * 8);
    meta[t] = *reinterpret_cast<const int*>(wl + L::META + t * 256 + lane * 4);
    const _Float16 sc =
        *reinterpret_cast<const _Float16*>(wl + L::SCALES + t * 32 + (lane & 15) * 2);
    s2[t] = half2v{sc, sc};
  }
  const half2v c0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const half2v c1 = {(_Float16)-72.0f, (_Float16)-72.0f};
  // fragment pairs (2h, i), (2h+1, i) of group g = h*MT + i, read one group ahead
  half8 ar[2][2];
  ar[0][0] = *reinterpret_cast<const half8*>(xb + aoff[0]);
  ar[0][1] = *reinterpret_cast<const half8*>(xb + aoff[1]);
  half8 b[2][NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) b[0][t] = dequant_scaled(wv[t].x, c0, c1, s2[t], magic);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int g = h * MT + i;
#pragma unroll
      for (int q = g; q < NVL; q += G) dma.issue(q);
      if (g + 1 < G) {
        const int gh = (g + 1) / MT, gi = (g + 1) % MT;
        ar[(g + 1) & 1][0] = *reinterpret_cast<const half8*>(xb + aoff[2 * gh] + gi * 4096);
        ar[(g + 1) & 1][1] = *reinterpret_cast<const half8*>(xb + aoff[2 * gh + 1] + gi * 4096);
      }
      if (h == 0) {
#pragma unroll
        for (int t = i; t < NTW; t += MT) b[1][t] = dequant_scaled(wv[t].y, c0, c1, s2[t], magic);
      }
      const half16 xbv = __builtin_shufflevector(ar[g & 1][0], ar[g & 1][1], 0, 1, 2, 3, 4, 5, 6,
                                                 7, 8, 9, 10, 11, 12, 13, 14, 15);
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        if (h == 0)
          acc[i][t] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(b[0][t], xbv, acc[i][t], meta[t], 0, 0);
        else
          acc[i][t] = __builtin_amdgcn_smfmac_f32_16x16x64_f16(b[1][t], xbv, acc[i][t], meta[t], 0, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One k-block of the fp16 baseline: weight fragments come straight from LDS (no
// unpacking); same group pipeline as the packed formats.
template <int MT, int NTW, class DP>
__device__ __forceinline__ void compute_kblock_fp16(const char* xb, const char* wl,
                                                    float4v (&acc)[MT][NTW],
                                                    const uint32_t (&aoff)[4], int lane,
                                                    const DP& dma) {
  constexpr int G = 4 * MT;
  constexpr int NVL = DP::NV;
  constexpr int PF = 3;
  half8 ar[PF + 1];
#pragma unroll
  for (int g = 0; g < PF; ++g)
    if (g < G) ar[g] = *reinterpret_cast<const half8*>(xb + aoff[g / MT] + (g % MT) * 4096);
  half8 b[2][NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t)
    b[0][t] = *reinterpret_cast<const half8*>(wl + (t * 4) * 1024 + lane * 16);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int g = j * MT + i;
#pragma unroll
      for (int q = g; q < NVL; q += G) dma.issue(q);
      if (g + PF < G) {
        const int gj = (g + PF) / MT, gi = (g + PF) % MT;
        ar[(g + PF) % (PF + 1)] = *reinterpret_cast<const half8*>(xb + aoff[gj] + gi * 4096);
      }
      if (j < 3) {
#pragma unroll
        for (int t = i; t < NTW; t += MT)
          b[(j + 1) & 1][t] = *reinterpret_cast<const half8*>(wl + (t * 4 + j + 1) * 1024 + lane * 16);
      }
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[j & 1][t], ar[g % (PF + 1)],
                                                          acc[i][t], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One k-block with fp8 activations.  The weights enter the matrix instruction as the
// exact E4M3 integers q - z, so the group scale cannot ride on them (3 mantissa bits):
// each (row tile, column tile) gets one v_mfma_scale_f32_16x16x128_f8f6f4 over the whole
// 128-row block (unit E8M0 scales) into a temporary, then acc += s * g in fp32 with the
// scales of the lane's four output columns.  Lane (l%16, q = l/16) holds k-slot 8j + e
// = row 32j + 8q + e of the block in both operands: the repacked word j of the weights
// and the activation bytes at 32j + 8q of its row.  Column tiles are the outer loop: the
// unpacking of tile t + 1 overlaps the matrix instructions of tile t.
template <int MT, int NTW, int MODE, class DP>
__device__ __forceinline__ void compute_kblock_fp8(const char* xb, const char* wl,
                                                   float4v (&acc)[MT][NTW],
                                                   const uint32_t (&aoff)[4], int lane,
                                                   uint32_t magic,
                                                   const DP& dma) {
  typedef WLds<NTW, MODE> L;
  constexpr int NVL = DP::NV;
  constexpr int G = NTW;  // groups per k-block: one per column tile
  int8v xa[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 v = *reinterpret_cast<const uint2*>(xb + aoff[j] + i * 2048);
      xa[i][2 * j] = (int)v.x;
      xa[i][2 * j + 1] = (int)v.y;
    }
  u32x4 wv[NTW];
  half2v c0[NTW], c1[NTW];
  float4v sc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    wv[t] = *reinterpret_cast<const u32x4*>(wl + t * 1024 + lane * 16);
    int zq = 8;
    if (mode_asym(MODE)) {
      const int c = lane & 15;
      const uint32_t zw = *reinterpret_cast<const uint32_t*>(wl + L::ZEROS + t * 8 + (c >> 3) * 4);
      zq = (int)((zw >> (4 * (c & 7))) & 15u);
    }
    const _Float16 a0 = (_Float16)(float)(-1024 - zq);
    const _Float16 a1 = (_Float16)(float)(-64 - zq);
    c0[t] = half2v{a0, a0};
    c1[t] = half2v{a1, a1};
    const uint2 s4 = *reinterpret_cast<const uint2*>(wl + L::SCALES + t * 32 + 8 * (lane >> 4));
    const half2v s01 = __builtin_bit_cast(half2v, s4.x), s23 = __builtin_bit_cast(half2v, s4.y);
    sc[t] = float4v{(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
  }
  auto unpack = [&](int t) {
    int8v b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 v = dequant_fp8(wv[t][j], c0[t], c1[t], magic);
      b[2 * j] = (int)v.x;
      b[2 * j + 1] = (int)v.y;
    }
    return b;
  };
  // group t: unpack tile t + 1, the matrix instructions of tile t, and the rescale of
  // tile t - 1 (whose products were issued one group earlier, so nothing waits on them)
  int8v b[2];
  float4v g[2][MT];
  b[0] = unpack(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t <= NTW; ++t) {
    if (t < NTW) {
#pragma unroll
      for (int q = t; q < NVL; q += G) dma.issue(q);
    }
    if (t + 1 < NTW) b[(t + 1) & 1] = unpack(t + 1);
    if (t < NTW) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        g[t & 1][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            b[t & 1], xa[i], float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
    }
    if (t >= 1) {
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[i][t - 1] += sc[t - 1] * g[(t - 1) & 1][i];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 8 codes of one repacked word -> the 8 exact bf16 values 128 + q (rows 0..7, the k order of
// the fp16 fragment): every nibble moved to bits 0-3 of its half and or-ed into the bits of
// 128 (bf16 keeps 7 mantissa bits, so the fp16 route through 1024 + 16q does not apply).
// Plain C: the compiler then knows these values feed a matrix instruction.
__device__ __forceinline__ bf16x8 codes_bf16(uint32_t w) {
  const uint32_t magic = 0x43004300u;
  const u32x4 r = {(w & 0x000F000Fu) | magic, ((w >> 4) & 0x000F000Fu) | magic,
                   ((w >> 8) & 0x000F000Fu) | magic, ((w >> 12) & 0x000F000Fu) | magic};
  return __builtin_bit_cast(bf16x8, r);
}

// One k-block with bf16 activations: the matrix instructions (v_mfma_f32_16x16x32_bf16)
// see the exact 128 + q, and per (row tile, column tile) the block's partial sum g is
// rescaled in fp32: acc += s (g - (128 + z) xs), with xs the sum of the lane's activation
// row over the block, taken on the matrix cores against a ones operand (the same four
// values in every lane of a row).  Weights stay exact integers and the scale applies once
// in fp32.  Software pipeline as for fp8: group t unpacks tile t + 1, runs the matrix
// instructions of tile t and rescales tile t - 1.
template <int MT, int NTW, int MODE, class DP>
__device__ __forceinline__ void compute_kblock_bf16(const char* xb, const char* wl,
                                                    float4v (&acc)[MT][NTW],
                                                    const uint32_t (&aoff)[4], int lane,
                                                    const DP& dma) {
  typedef WLds<NTW, MODE> L;
  constexpr int NVL = DP::NV;
  constexpr int G = NTW;  // groups per k-block: one per column tile
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                       0x3F803F80u});
  bf16x8 xa[MT][4];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      xa[i][j] = *reinterpret_cast<const bf16x8*>(xb + aoff[j] + i * 4096);
  float xs[MT];
  {
    float4v v[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) v[i] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < MT; ++i)
        v[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, xa[i][j], v[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < MT; ++i) xs[i] = v[i][0];
  }
  u32x4 wv[NTW];
  float4v sc[NTW], so[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    wv[t] = *reinterpret_cast<const u32x4*>(wl + t * 1024 + lane * 16);
    // the lane's four columns 16t + 4(lane/16) + r: scales and offsets 128 + z
    const uint2 s4 = *reinterpret_cast<const uint2*>(wl + L::SCALES + t * 32 + 8 * (lane >> 4));
    const half2v s01 = __builtin_bit_cast(half2v, s4.x), s23 = __builtin_bit_cast(half2v, s4.y);
    sc[t] = float4v{(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
    float4v off = {136.f, 136.f, 136.f, 136.f};
    if constexpr (mode_asym(MODE)) {
      const uint2 zw = *reinterpret_cast<const uint2*>(wl + L::ZEROS + t * 8);
      const uint32_t z16 = (((lane >> 4) < 2 ? zw.x : zw.y) >> (16 * ((lane >> 4) & 1))) & 0xFFFFu;
#pragma unroll
      for (int r = 0; r < 4; ++r) off[r] = (float)(128 + (int)((z16 >> (4 * r)) & 15u));
    }
    so[t] = sc[t] * off;
  }
  bf16x8 b[2][4];
  float4v g[2][MT];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[0][j] = codes_bf16(wv[0][j]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t <= NTW; ++t) {
    if (t < NTW) {
#pragma unroll
      for (int q = t; q < NVL; q += G) dma.issue(q);
    }
    if (t + 1 < NTW) {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[(t + 1) & 1][j] = codes_bf16(wv[t + 1][j]);
    }
    if (t < NTW) {
#pragma unroll
      for (int i = 0; i < MT; ++i) g[t & 1][i] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          g[t & 1][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[t & 1][j], xa[i][j],
                                                                g[t & 1][i], 0, 0, 0);
    }
    if (t >= 1) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
        acc[i][t - 1] += sc[t - 1] * g[(t - 1) & 1][i] - so[t - 1] * xs[i];
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One k-block of MXFP4 weights: the codes go to the block-scaled matrix instruction as
// they are (E2M1 operand A), with the lane's E8M0 byte as its scale, and the fp8 rows of
// X as operand B (unit scale); the instruction applies the scales of the 32-row blocks
// itself, so there is no unpacking and no rescaling.  The two operands place K
// differently: an FP4 lane (l/16 = g) holds rows 32g .. 32g+31 in order (so its scale
// byte covers exactly its own codes: lane l of the 1 KiB block holds column l%16, rows
// 32g .. +31), while an FP8 lane holds rows 16g .. 16g+15 in its first 16 bytes and
// 64+16g .. +15 in its last 16 (measured with one-hot activations).  The X fragment of
// lane l is therefore chunks g and 4+g of row 16i + l%16 of the swizzled tile (two
// 16-byte reads).  The loads of a later k-block are spread over the row tiles' groups.
template <int MT, int NTW, int MODE, class DP>
__device__ __forceinline__ void compute_kblock_mx(const char* xb, const char* wl,
                                                  float4v (&acc)[MT][NTW],
                                                  const uint32_t (&aoff)[4], int lane,
                                                  const DP& dma) {
  typedef WLds<NTW, MODE> L;
  constexpr int NVL = DP::NV;
  int8v b[NTW];
  int sc[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(wl + t * 1024 + lane * 16);
    b[t] = int8v{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
    sc[t] = (int)*reinterpret_cast<const uint8_t*>(wl + L::SCALES + t * 64 + lane);
  }
  auto frag = [&](int i) {
    const u32x4 lo = *reinterpret_cast<const u32x4*>(xb + aoff[0] + i * 2048);
    const u32x4 hi = *reinterpret_cast<const u32x4*>(xb + aoff[1] + i * 2048);
    return int8v{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  int8v xa[2];
  xa[0] = frag(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int q = i; q < NVL; q += MT) dma.issue(q);
    if (i + 1 < MT) xa[(i + 1) & 1] = frag(i + 1);
#pragma unroll
    for (int t = 0; t < NTW; ++t)
      acc[i][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          b[t], xa[i & 1], acc[i][t], 4, 0, 0, sc[t], 0, 127);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// vmcnt(n) with the other counters left alone (gfx9 encoding)
__device__ __forceinline__ constexpr int vmcnt_enc(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}
// bf16 outputs: round to nearest even from fp32 (finite values)
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_b2(float a, float b) {
  return bf16_bits(a) | (bf16_bits(b) << 16);
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
  // integer division runs on the vector unit; the results are uniform, say so
  tm = __builtin_amdgcn_readfirstlane(first + r % gm);
  tn = __builtin_amdgcn_readfirstlane(r / gm);
}

// Y store of row tiles i0 .. i0 + NI - 1 of a finished tile tt: lane holds row 16i +
// lane%16 and the four columns 16t + 4(lane/16) .. +3 of each of the wave's NTW column
// tiles.
template <int MT, int NTW, int NI, int NWV>
__device__ __forceinline__ void store_rows(uint16_t* __restrict__ Y, const TiledArgs& a, int tt,
                                           int i0, int wave, int lane,
                                           const float4v (&acc)[NI][NTW]) {
  constexpr int BM = 16 * MT;
  constexpr int BN = NWV * 16 * NTW;
  int tm, tn;
  tile_coords(tt, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
  const int m0 = tm * BM;
  const int rows = a.M - m0 < BM ? a.M - m0 : BM;
  const rsrc_t ry = make_rsrc(Y + (size_t)m0 * a.N, (uint32_t)((size_t)rows * a.N * 2));
  const int t_first = tn * (BN / 16) + wave * NTW;
  const int ntiles16 = a.N / 16;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (t_first + t >= ntiles16) break;  // wave-uniform
#pragma unroll
    for (int ii = 0; ii < NI; ++ii) {
      const int r = 16 * (i0 + ii) + (lane & 15);
      const uint32_t off = r < rows ? (uint32_t)(((size_t)r * a.N + (t_first + t) * 16 +
                                                  4 * (lane >> 4)) * 2)
                                    : kOutOfRange;
      // fp8 activations, or rows rewritten in fp16: the scale of the row, applied once to
      // the finished sum
      const float xs = (a.xscale != nullptr && r < rows) ? a.xscale[m0 + r] : 1.0f;
      const float4v o = a.xscale != nullptr ? acc[ii][t] * xs : acc[ii][t];
      typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 v = a.out_bf16 ? u32x2{pack_b2(o[0], o[1]), pack_b2(o[2], o[3])}
                                 : u32x2{pack_h2(o[0], o[1]), pack_h2(o[2], o[3])};
      __builtin_amdgcn_raw_buffer_store_b64(v, ry, off, 0u, 0);
    }
  }
}
template <int MT, int NTW, int NWV>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ Y, const TiledArgs& a, int tt,
                                           int wave, int lane, const float4v (&acc)[MT][NTW]) {
  store_rows<MT, NTW, MT, NWV>(Y, a, tt, 0, wave, lane, acc);
}

// Byte offset of one lane's float4 of (row tile i, column tile t) inside a partial piece.
template <int MT, int NTW>
__device__ __forceinline__ uint32_t piece_off(int wave, int i, int t, int lane) {
  return (uint32_t)((((wave * MT + i) * NTW + t) * 64 + lane) * 16);
}

template <int MT, int NTW, int NS, int MODE, int NWV>
__global__ __launch_bounds__(64 * NWV) void tiled_kernel(
    const uint16_t* __restrict__ X, const uint32_t* __restrict__ W,
    const uint16_t* __restrict__ Sp, const uint32_t* __restrict__ Zp, uint16_t* __restrict__ Y,
    float* __restrict__ part, TiledArgs a) {
  constexpr int BM = 16 * MT;
  constexpr int BN = NWV * 16 * NTW;
  constexpr bool F8 = mode_fp8(MODE);
  constexpr int XBUF = BM * (F8 ? 128 : 256);  // one k-block of the activation tile
  constexpr int NSTAGE = NS;       // LDS pipeline stages
  constexpr int AHEAD = NS - 1;    // k-blocks in flight ahead of the one computed
  constexpr int PIECE = BM * BN;   // floats of one partial tile
  constexpr int STAGE = XBUF + NWV * WLds<NTW, MODE>::BYTES;  // LDS bytes of one stage
  typedef DmaPlan<MT, NTW, MODE, NWV> DP;
  constexpr int NV = DP::NV;  // loads per stage per thread
  constexpr int NX = DP::NX;  // activation loads per stage per thread
  __shared__ __attribute__((aligned(1024))) char lds[NSTAGE * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Gk = a.K / KBLK;
  const int ntiles16 = a.N / 16;
  const uint32_t magic = 0x64006400u;
  // per-lane LDS offsets of the fragment reads of k-step j (row tile 0; row tile i
  // adds 16 rows = 4096 bytes): row lane%16, chunk 4j + lane/16
  // (fp8: the 8 bytes at 32j + 8(lane/16) of row lane%16, row tile i adds 2048 bytes)
  uint32_t aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    aoff[j] = MODE == W_MX4 ? swz8(lane & 15, (lane >> 4) + 4 * (j & 1))
              : F8          ? swz8(lane & 15, 2 * j + (lane >> 5)) + 8 * ((lane >> 4) & 1)
                            : swz(lane & 15, 4 * j + (lane >> 4));

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
    constexpr int XB = F8 ? 1 : 2;  // bytes per activation
    const u32x4 rx = rsrc_words(reinterpret_cast<const char*>(X) + (size_t)m0 * a.K * XB,
                                (uint32_t)((size_t)rows * a.K * XB));
    uint32_t xoff[NX];
#pragma unroll
    for (int c = 0; c < NX; ++c) {
      if constexpr (F8) {
        // lane L: row 8(wave*NX + c) + L/8, the global chunk stored at position L%8
        const int r = 8 * (wave * NX + c) + (lane >> 3);
        const int cg = (lane & 7) ^ ((r >> 1) & 7);
        xoff[c] = r < rows ? (uint32_t)((size_t)r * a.K + 16 * cg) : kOutOfRange;
      } else {
        const int r = 4 * (wave * NX + c) + (lane >> 4);
        const int cg = (lane & 15) ^ (r & 15);  // global chunk stored at position lane%16
        xoff[c] = r < rows ? (uint32_t)(((size_t)r * a.K + 8 * cg) * 2) : kOutOfRange;
      }
    }
    const int t_first = tn * (BN / 16) + wave * NTW;  // first 16-column tile of this wave
    int nvalid = ntiles16 - t_first;
    nvalid = nvalid < 0 ? 0 : (nvalid > NTW ? NTW : nvalid);
    WSrc<NTW> R;
    constexpr int SH = mode_scale64(MODE) ? 2 : 1;  // 32-byte scale rows per block
    if (MODE != W_FP16) {
      // scales: lane L < 8*SH*NTW loads bytes 4(L % 8SH) .. +3 of tile L / 8SH's row(s)
      R.s = rsrc_words(Sp + (size_t)t_first * Gk * 16 * SH, (uint32_t)(nvalid * Gk * 32 * SH));
      const int ts = lane / (8 * SH);
      R.so = (lane < 8 * SH * NTW && ts < nvalid)
                 ? (uint32_t)(ts * Gk * 32 * SH + (lane % (8 * SH)) * 4)
                 : kOutOfRange;
    } else {
      R.s = rsrc_words(W, 0);  // no scales
      R.so = kOutOfRange;
    }
    if (MODE == W_FP16) {
      // fp16 rows of the wave's columns: lane L of the load for (tile t, k-step j) reads
      // 16 bytes of row 16t + L%16 at column 128kb + 32j + 8(L/16)
      R.w = rsrc_words(reinterpret_cast<const char*>(W) + (size_t)t_first * 16 * a.K * 2,
                       (uint32_t)((size_t)nvalid * 16 * a.K * 2));
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        R.wo[t] = t < nvalid ? (uint32_t)(((16 * t + (lane & 15)) * (size_t)a.K + 8 * (lane >> 4)) * 2)
                             : kOutOfRange;
      R.z = R.s;
      R.zo = kOutOfRange;
    } else if (MODE == W_SP24) {
      // kept codes (512 B per block; lanes 32c.. load tiles 2c, 2c+1) and positions
      // (256 B per block, passed in Zp; lane L loads tile L/16)
      R.w = rsrc_words(reinterpret_cast<const char*>(W) + (size_t)t_first * Gk * 512,
                       (uint32_t)(nvalid * Gk * 512));
      R.z = rsrc_words(reinterpret_cast<const char*>(Zp) + (size_t)t_first * Gk * 256,
                       (uint32_t)(nvalid * Gk * 256));
#pragma unroll
      for (int c = 0; c < NTW / 2; ++c) {
        const int t = 2 * c + (lane >> 5);
        R.wo[c] = t < nvalid ? (uint32_t)(t * Gk * 512 + (lane & 31) * 16) : kOutOfRange;
      }
      const int tz = lane >> 4;
      R.zo = tz < nvalid ? (uint32_t)(tz * Gk * 256 + (lane & 15) * 16) : kOutOfRange;
    } else {
      R.w = rsrc_words(reinterpret_cast<const char*>(W) + (size_t)t_first * Gk * 1024,
                       (uint32_t)(nvalid * Gk * 1024));
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        R.wo[t] = t < nvalid ? (uint32_t)(t * Gk * 1024 + lane * 16) : kOutOfRange;
      if (mode_asym(MODE)) {
        // zero-points: lane L < 2*SH*NTW loads word L % 2SH of tile L / 2SH
        R.z = rsrc_words(reinterpret_cast<const char*>(Zp) + (size_t)t_first * Gk * 8 * SH,
                         (uint32_t)(nvalid * Gk * 8 * SH));
        const int tz = lane / (2 * SH);
        R.zo = (lane < 2 * SH * NTW && tz < nvalid)
                   ? (uint32_t)(tz * Gk * 8 * SH + (lane % (2 * SH)) * 4)
                   : kOutOfRange;
      } else {
        R.z = R.s;
        R.zo = kOutOfRange;
      }
    }
    // zero-size resources: loads past the segment return zeros without a memory
    // request (their LDS destination still receives zeros), so the number of loads
    // in flight is the same in every iteration and the wait counts below are static
    const u32x4 rx0 = rsrc_words(X, 0);
    WSrc<NTW> R0 = R;
    R0.w = rsrc_words(W, 0);
    R0.s = rsrc_words(W, 0);
    R0.z = R0.s;

#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t) acc[i][t] = float4v{0.f, 0.f, 0.f, 0.f};

    const int nk = kb1 - kb0;
    const uint32_t lds0 = lds_addr(lds);
    const uint32_t wl0 = lds0 + XBUF + wave * WLds<NTW, MODE>::BYTES;  // this wave's weight slot, stage 0
    // every wave is done with the LDS buffers of the previous segment
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // prologue: k-blocks kb0 .. kb0 + AHEAD - 1 in flight
#pragma unroll
    for (int p = 0; p < AHEAD; ++p) {
      const bool live = p < nk;
      DP plan;
      plan.rx = live ? rx : rx0;
#pragma unroll
      for (int c = 0; c < NX; ++c) plan.xoff[c] = xoff[c];
      plan.R = live ? R : R0;
      plan.xdst = lds0 + p * STAGE;
      plan.wdst = wl0 + p * STAGE;
      plan.wave = wave;
      plan.kb = kb0 + p;
#pragma unroll
      for (int q = 0; q < NV; ++q) plan.issue(q);
    }
    __builtin_amdgcn_sched_barrier(0);

    // step d of the ring handles k-block kbi, held in stage d; k-block kbi + AHEAD is
    // issued into stage (d + AHEAD) % NS, one load per fragment group of the compute.
    // At the wait, the loads of kbi .. kbi + AHEAD - 1 are in flight (NV per stage,
    // oldest first); after it, every wave's loads of kbi have landed once all waves
    // pass the barrier, and every wave has finished reading the stage to be refilled.
    auto step = [&](int d, int kbi, bool issue_live) {
      d = __builtin_amdgcn_readfirstlane(d);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(vmcnt_enc((AHEAD - 1) * NV));
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
      const int dn = (d + AHEAD) % NSTAGE;
      DP plan;
      plan.rx = issue_live ? rx : rx0;
#pragma unroll
      for (int c = 0; c < NX; ++c) plan.xoff[c] = xoff[c];
      plan.R = issue_live ? R : R0;
      plan.xdst = lds0 + dn * STAGE;
      plan.wdst = wl0 + dn * STAGE;
      plan.wave = wave;
      plan.kb = kbi + AHEAD;
      if constexpr (MODE == W_FP16)
        compute_kblock_fp16<MT, NTW>(lds + d * STAGE,
                                     lds + d * STAGE + XBUF + wave * WLds<NTW, MODE>::BYTES, acc,
                                     aoff, lane, plan);
      else if constexpr (MODE == W_SP24)
        compute_kblock_sp24<MT, NTW>(lds + d * STAGE,
                                     lds + d * STAGE + XBUF + wave * WLds<NTW, MODE>::BYTES, acc,
                                     aoff, lane, magic, plan);
      else if constexpr (MODE == W_MX4)
        compute_kblock_mx<MT, NTW, MODE>(lds + d * STAGE,
                                         lds + d * STAGE + XBUF + wave * WLds<NTW, MODE>::BYTES,
                                         acc, aoff, lane, plan);
      else if constexpr (mode_bf16(MODE))
        compute_kblock_bf16<MT, NTW, MODE>(lds + d * STAGE,
                                           lds + d * STAGE + XBUF + wave * WLds<NTW, MODE>::BYTES,
                                           acc, aoff, lane, plan);
      else if constexpr (F8)
        compute_kblock_fp8<MT, NTW, MODE>(lds + d * STAGE,
                                          lds + d * STAGE + XBUF + wave * WLds<NTW, MODE>::BYTES,
                                          acc, aoff, lane, magic, plan);
      else
        compute_kblock<MT, NTW, MODE>(lds + d * STAGE,
                                      lds + d * STAGE + XBUF + wave * WLds<NTW, MODE>::BYTES, acc,
                                      aoff, lane, magic, plan);
      __builtin_amdgcn_sched_barrier(0);
    };
    // one k-block per trip with a rotating stage index: stages are LDS addresses, so
    // nothing needs unrolling, and the accumulators keep their registers across the
    // back-edge (an unrolled body made the allocator shuffle them every trip)
    int d = 0;
#pragma nounroll
    for (int i = 0; i < nk; ++i) {
      step(d, kb0 + i, i + AHEAD < nk);
      d = d + 1 == NS ? 0 : d + 1;
    }
    // drain: no load of this segment is left in flight
    __builtin_amdgcn_s_waitcnt(0);
  };

  auto store_y = [&](int tt, const float4v (&acc)[MT][NTW]) {
    store_tile<MT, NTW, NWV>(Y, a, tt, wave, lane, acc);
  };


  // ---- data-parallel rounds: tile it*grid + w, full K ----
  for (int it = 0; it < a.dp_rounds; ++it) {
    const int tt = it * a.grid + w;
    float4v acc[MT][NTW];
    run_segment(tt, 0, Gk, acc);
    store_y(tt, acc);
  }
  if (a.sk_units == 0) return;

  // ---- stream-K stripe [u0, u1) over the remaining tiles' (tile, k-block) units ----
  // (32-bit bookkeeping, bounded by the plan; every quantity is uniform)
  const uint32_t U = (uint32_t)a.sk_per_wg;
  const uint32_t nunits = (uint32_t)a.sk_units;
  const uint32_t u0 = (uint32_t)w * U;
  const uint32_t u1 = u0 + U < nunits ? u0 + U : nunits;
  for (uint32_t u = u0; u < u1;) {
    const int tl = __builtin_amdgcn_readfirstlane((int)(u / (uint32_t)Gk));  // tile in the stream-K part
    const int kb0 = __builtin_amdgcn_readfirstlane((int)(u - (uint32_t)tl * Gk));
    const uint32_t rest = u1 - u;
    const int kb1 = rest < (uint32_t)(Gk - kb0) ? kb0 + (int)rest : Gk;
    const int tt = a.dp_rounds * a.grid + tl;
    float4v acc[MT][NTW];
    run_segment(tt, kb0, kb1, acc);
    const bool first_seg = (u == u0);
    u += (uint32_t)(kb1 - kb0);
    if (kb0 == 0 && kb1 == Gk) {
      store_y(tt, acc);
      continue;
    }
    // a tile cut by a stripe boundary: store this piece (two slots per workgroup: its
    // first and its last segment); the second pass sums the pieces and writes Y
    const int slot = __builtin_amdgcn_readfirstlane(2 * w + (first_seg ? 0 : 1));
    const rsrc_t rp = make_rsrc(part + (size_t)slot * PIECE, PIECE * 4);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][t]), rp,
                                               piece_off<MT, NTW>(wave, i, t, lane), 0u, 0);
  }
}

// Second pass of the stream-K split: one workgroup per (tile of the stream-K part, row
// tile of 16 rows); a tile cut into pieces by stripe boundaries gets the pieces summed in
// stripe order (a fixed order, so results are bitwise reproducible) and written to Y.
// Tiles done by a single workgroup were stored by it directly.  The loads of up to four
// pieces are in flight together.
template <int MT, int NTW, int NWV>
__global__ __launch_bounds__(64 * NWV) void tiled_fixup_kernel(const float* __restrict__ part,
                                                               uint16_t* __restrict__ Y,
                                                               TiledArgs a) {
  constexpr int PIECE = 16 * MT * NWV * 16 * NTW;
  constexpr int CH = 4;  // pieces per batch of loads
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tl = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / MT));
  const int i = __builtin_amdgcn_readfirstlane((int)(blockIdx.x % MT));
  const uint32_t Gk = (uint32_t)(a.K / KBLK);
  const uint32_t U = (uint32_t)a.sk_per_wg;
  const int w_first = __builtin_amdgcn_readfirstlane((int)(((uint32_t)tl * Gk) / U));
  const int w_last = __builtin_amdgcn_readfirstlane((int)(((uint32_t)(tl + 1) * Gk - 1) / U));
  if (w_first == w_last) return;
  float4v sum[1][NTW];
  for (int wp = w_first; wp <= w_last; wp += CH) {
    float4v v[CH][NTW];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int wq = wp + c;
      const bool live = wq <= w_last;  // uniform; past the last piece: zero-size reads
      const int first_tile_of_wq = (int)(((uint32_t)wq * U) / Gk);
      const int sl = __builtin_amdgcn_readfirstlane(
          live ? 2 * wq + (tl == first_tile_of_wq ? 0 : 1) : 0);
      const rsrc_t rp = make_rsrc(part + (size_t)sl * PIECE, live ? PIECE * 4 : 0);
#pragma unroll
      for (int t = 0; t < NTW; ++t)
        v[c][t] = __builtin_bit_cast(
            float4v, __builtin_amdgcn_raw_buffer_load_b128(rp, piece_off<MT, NTW>(wave, i, t, lane),
                                                           0u, 0));
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (wp + c > w_last) break;  // uniform
#pragma unroll
      for (int t = 0; t < NTW; ++t) sum[0][t] = wp + c == w_first ? v[c][t] : sum[0][t] + v[c][t];
    }
  }
  store_rows<MT, NTW, 1, NWV>(Y, a, a.dp_rounds * a.grid + tl, i, wave, lane, sum);
}

typedef void (*TiledFn)(const uint16_t*, const uint32_t*, const uint16_t*, const uint32_t*,
                        uint16_t*, float*, TiledArgs);
typedef void (*FixupFn)(const float*, uint16_t*, TiledArgs);

struct TVariant {
  int MT, NTW, NS, NWV;  // row tiles, column tiles per wave, pipeline stages, waves
  TiledFn sym, asym, sp24, f16, sym64, asym64, sym8, asym8, mx4, symb, asymb;
  FixupFn fixup;
  const char* name;
};

// fp8 activations need an even number of 16-row tiles (one 1 KiB load covers 8 rows)
template <int MT, int NTW, int NS, int MODE, int NWV = WAVES>
constexpr TiledFn fp8_tiled() {
  if constexpr (MT % 2 == 0) return tiled_kernel<MT, NTW, NS, MODE, NWV>;
  else return nullptr;
}
// the 2:4 format's loads are laid out for four column tiles per wave (two tiles' kept codes
// per 16-byte load, all four tiles' positions in one)
template <int MT, int NTW, int NS>
constexpr TiledFn sp24_tiled() {
  if constexpr (NTW == 4) return tiled_kernel<MT, NTW, NS, W_SP24, WAVES>;
  else return nullptr;
}

#define W4A16_TILED(MT, NTW, NS, NAME)                                                       \
  TVariant {                                                                               \
    MT, NTW, NS, WAVES, tiled_kernel<MT, NTW, NS, W_SYM, WAVES>,                            \
        tiled_kernel<MT, NTW, NS, W_ASYM, WAVES>, sp24_tiled<MT, NTW, NS>(), nullptr,       \
        tiled_kernel<MT, NTW, NS, W_SYM64, WAVES>, tiled_kernel<MT, NTW, NS, W_ASYM64, WAVES>, \
        fp8_tiled<MT, NTW, NS, W_SYM8>(), fp8_tiled<MT, NTW, NS, W_ASYM8>(),                \
        fp8_tiled<MT, NTW, NS, W_MX4>(), tiled_kernel<MT, NTW, NS, W_SYMB, WAVES>,          \
        tiled_kernel<MT, NTW, NS, W_ASYMB, WAVES>, tiled_fixup_kernel<MT, NTW, WAVES>, NAME \
  }
// eight waves (two per SIMD) sharing a BM-row activation tile, each with the same 16*NTW
// columns of work as in the four-wave variants: the packed formats except 2:4 and bf16
// activations (their X fragments, partial sums and rescale do not fit two waves).  The
// fp8-activation INT4 modes only with two column tiles per wave (with four, their
// unpacking and rescale do not fit the registers of two waves per SIMD: the main loop
// spills).
template <int MT, int NTW, int NS, int MODE>
constexpr TiledFn fp8_tiled_w8() {
  if constexpr (NTW <= 2) return fp8_tiled<MT, NTW, NS, MODE, 8>();
  else return nullptr;
}
#define W4A16_TILED_W8(MT, NTW, NS, NAME)                                                    \
  TVariant {                                                                               \
    MT, NTW, NS, 8, tiled_kernel<MT, NTW, NS, W_SYM, 8>, tiled_kernel<MT, NTW, NS, W_ASYM, 8>, \
        nullptr, nullptr, tiled_kernel<MT, NTW, NS, W_SYM64, 8>,                            \
        tiled_kernel<MT, NTW, NS, W_ASYM64, 8>, fp8_tiled_w8<MT, NTW, NS, W_SYM8>(),        \
        fp8_tiled_w8<MT, NTW, NS, W_ASYM8>(), fp8_tiled<MT, NTW, NS, W_MX4, 8>(), nullptr,  \
        nullptr, tiled_fixup_kernel<MT, NTW, 8>, NAME                                       \
  }
// the fp16 baseline moves four times the weight bytes: its own LDS-sized tiles
#define W4A16_TILED_F16(MT, NTW, NS, NAME)                                                    \
  TVariant {                                                                               \
    MT, NTW, NS, WAVES, nullptr, nullptr, nullptr, tiled_kernel<MT, NTW, NS, W_FP16, WAVES>, \
        nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,                      \
        tiled_fixup_kernel<MT, NTW, WAVES>, NAME                                            \
  }

const TVariant kTiled[] = {
    W4A16_TILED(8, 4, 3, "tiled_bm128_bn256_s3"),
    W4A16_TILED(4, 4, 4, "tiled_bm64_bn256_s4"),
    W4A16_TILED(4, 4, 3, "tiled_bm64_bn256_s3"),
    W4A16_TILED(2, 4, 4, "tiled_bm32_bn256_s4"),
    W4A16_TILED(1, 4, 4, "tiled_bm16_bn256_s4"),
    W4A16_TILED(8, 2, 3, "tiled_bm128_bn128_s3"),
    W4A16_TILED_W8(8, 4, 2, "tiled_bm128_bn512_w8_s2"),
    W4A16_TILED_W8(8, 2, 3, "tiled_bm128_bn256_w8_s3"),
    W4A16_TILED(4, 2, 4, "tiled_bm64_bn128_s4"),
};
constexpr int kNumTiled = sizeof(kTiled) / sizeof(kTiled[0]);
const TVariant kTiledF16[] = {
    W4A16_TILED_F16(8, 2, 2, "tiled_f16_bm128_bn128_s2"),
    W4A16_TILED_F16(4, 2, 3, "tiled_f16_bm64_bn128_s3"),
};
constexpr int kNumTiledF16 = sizeof(kTiledF16) / sizeof(kTiledF16[0]);

// the kernel of a variant for a weight format (nullptr where the variant does not run it)
TiledFn variant_fn(const TVariant& v, int mode) {
  return mode == W_ASYM     ? v.asym
         : mode == W_SP24   ? v.sp24
         : mode == W_FP16   ? v.f16
         : mode == W_SYM64  ? v.sym64
         : mode == W_ASYM64 ? v.asym64
         : mode == W_SYM8   ? v.sym8
         : mode == W_ASYM8  ? v.asym8
         : mode == W_MX4    ? v.mx4
         : mode == W_SYMB   ? v.symb
         : mode == W_ASYMB  ? v.asymb
         : mode == W_SYM    ? v.sym
                            : nullptr;
}

}  // namespace

int tiled_variant_count(int mode) { return mode == W_FP16 ? kNumTiledF16 : kNumTiled; }
const char* tiled_variant_name(int mode, int v) {
  if (v < 0 || v >= tiled_variant_count(mode)) return nullptr;
  return mode == W_FP16 ? kTiledF16[v].name : kTiled[v].name;
}

// A workgroup count between 224 and 256 that divides `tiles` exactly (the largest), or 0:
// with it every workgroup takes whole tiles, in equal numbers, and no tile is cut.
static long dp_grid(long tiles) {
  for (long g = 256; g >= 224; --g)
    if (tiles % g == 0) return g;
  return 0;
}

int tiled_make_plan(int M, int N, int K, int mode, int variant, int grid, TiledPlan* p) {
  // fp8 and bf16 activations: groups of 128 rows or more (one scale per 128-row block)
  if ((!mode_dense4(mode) && mode != W_SP24 && mode != W_FP16) || mode == W_SYMB64 ||
      mode == W_ASYMB64 || mode == W_SYM8G64 || mode == W_ASYM8G64)
    return -8;
  const bool f8 = mode_fp8(mode);
  const bool f16 = mode == W_FP16;
  const TVariant* table = f16 ? kTiledF16 : kTiled;
  const int count = f16 ? kNumTiledF16 : kNumTiled;
  // measured on MI355X: the 128-row tile wins from M = 128 on (more reuse of each
  // unpacked weight; 11% at M = 128 on 8192 x 28672); above 64 rows both tiles compute
  // 128 padded rows, so the 64-row tile (3-deep ring: 1-4% faster than 4-deep at
  // M = 48-64) is kept for M <= 64 only.  The fp16 baseline's table: 128 x 128 above
  // 64 rows, 64 x 128 up to 64.
  if (variant < 0) {
    variant = M > 64 ? 0 : (f16 ? 1 : 2);
    const bool dense16 = mode == W_SYM || mode == W_ASYM || mode == W_SYM64 || mode == W_ASYM64;
    const bool int4fp8 = mode == W_SYM8 || mode == W_ASYM8;
    const bool large = (long long)K * N >= (128LL << 20);
    // layers up to 128 Mi weights at 65-256 rows: 128 x 128 tiles, twice the tiles of
    // 128 x 256 for the 256 compute units (measured 1.04-1.14x at M = 128 and 1.02-1.06x at
    // M = 256 on 8192 x 10240, 5120 x 13824, 13824 x 5120, 4096 x 11008; slower on the
    // 235 Mi-weight layers and at M >= 1024; with fp8 activations 0.88x at M = 256 on
    // 8192 x 10240, so those keep 128 x 256)
    if (!f16 && mode != W_SP24 && !int4fp8 && M > 64 && M <= 256 &&
        (long long)K * N <= (128LL << 20))
      variant = 5;
    // 33-64 rows on layers up to 128 Mi weights: 64 x 128 tiles, four k-blocks deep
    // (measured 1.04-1.09x over 64 x 256 at M = 48 and 64 on 8192 x 10240, 5120 x 13824
    // and 13824 x 5120; slower on the 235 Mi-weight layers)
    if (variant == 2 && dense16 && (long long)K * N <= (128LL << 20)) variant = 8;
    // 128-row tiles would pad M by more than an eighth (M % 128 in 1..64, M < 512): 64-row
    // tiles instead (measured 1.05-1.26x faster at M = 192 on six 7B/70B-class layers, and
    // 1.08-1.18x slower at M = 256 / 384 where 128-row tiles pad nothing), except for the
    // packed formats with fp16 activations on layers of 128 Mi weights or more from 129
    // rows on, and on every layer above 384 rows, where the eight-wave 128-row tiles below
    // win despite the padding (1.05-1.26x at M = 160-448 on 8192 x 28672 and 28672 x 8192,
    // 1.10x at M = 448 on 8192 x 10240)
    // (MXFP4 and the 2:4 format keep 128-row tiles there on layers of 128 Mi weights or
    // more: 1.25-1.45x and 1.02-1.14x at M = 192 on 8192 x 28672 and 28672 x 8192)
    if (!f16 && M > 128 && M < 512 && M % 128 != 0 && M % 128 <= 64 &&
        !(dense16 && (large || M > 384)) && !((mode == W_MX4 || mode == W_SP24) && large))
      variant = 2;
    // MXFP4 takes the 64-row tiles as 64 x 128 up to 256 rows on every layer (1.08-1.21x
    // at M = 48-64 on the three 70B-class layers, 1.10x at M = 192 on 8192 x 10240; at
    // M = 320 there the 200 tiles of 64 x 256 in one round are 1.28x faster)
    if (variant == 2 && mode == W_MX4 && M <= 256) variant = 8;
    // MXFP4 has no skinny kernel: up to 32 rows take the 32-row tile; the 2:4 format
    // (automatically tiled from 17 rows on on large layers) takes 16-row tiles up to 16
    // rows and 32-row tiles up to 32 (the fastest tiles at M = 16 / 32 on 8192 x 28672)
    if (mode == W_MX4 && M <= 32) variant = 3;
    if (mode == W_SP24 && M <= 32) variant = M <= 16 ? 4 : 3;
    // Eight waves (two per SIMD): the second wave on each SIMD issues its unpacking and LDS
    // reads while the first one's MFMAs run.
    // fp16 activations: 128 x 512 tiles once they fill the 256 compute units at least twice
    // over, or in whole rounds of 224-256 workgroups (no stream-K stripes): measured
    // 1.06-1.11x at M = 2048-4096 on 8192 x 28672, 1.09-1.11x at M = 2048 / 4096 on
    // 28672 x 8192, 1.0-1.02x on 8192 x 10240; at M = 1024 on 8192 x 28672, 448 tiles as two
    // rounds of 224 workgroups: 1.10x, where 256 workgroups and stream-K stripes were 0.96x;
    // 0.88-0.93x at M = 256.  Otherwise, from one full round of 128 x 256 tiles on, the
    // same tiles with eight waves (32 columns each): 1.04x at M = 1024 on 28672 x 8192,
    // 1.01-1.03x on 8192 x 10240; on layers of 128 Mi weights or more also below a full
    // round (1.01-1.05x at M = 128-256 on 8192 x 28672 and 28672 x 8192).
    // MXFP4: 128 x 512 tiles in whole rounds only (1.04-1.18x at M = 1024 / 4096 on the
    // 235 Mi-weight layers; with stream-K stripes 0.86-0.93x), else 128 x 256 with eight
    // waves from a full round on (1.06x at M = 1024 and 4096 on 8192 x 10240).
    // fp8 activations (INT4 codes): no 128 x 512 eight-wave tiles (they spill); 128 x 256
    // with eight waves where those tiles make whole rounds of 256 (1.01-1.04x at M = 4096;
    // 0.90-0.93x at M = 1024 on 8192 x 28672 with its 896 tiles as four rounds of 224), or
    // number 200-511 (1.04x at M = 256 on 8192 x 28672 and at M = 1024 on 8192 x 10240).
    if (variant == 0 && (dense16 || int4fp8 || mode == W_MX4)) {
      const long long t8 = (long long)((M + 127) / 128) * ((N + 511) / 512);
      const long long t4 = (long long)((M + 127) / 128) * ((N + 255) / 256);
      if ((dense16 && (t8 >= 512 || dp_grid(t8) > 0)) || (mode == W_MX4 && dp_grid(t8) > 0))
        variant = 6;
      else if ((!int4fp8 && t4 >= 256) || (dense16 && large) ||
               (int4fp8 && (t4 % 256 == 0 || (t4 >= 200 && t4 < 512))))
        variant = 7;
    }
    if (!f16) {
      // a layer too small to give the chip a thousand (tile, k-block) units with these
      // tiles (3072 x 768: 72 at M = 128) runs on 16-row tiles instead, which gives
      // it 8x the units (measured 1.2-1.6x faster there)
      const TVariant& d = table[variant];
      const long long units = (long long)((M + 16 * d.MT - 1) / (16 * d.MT)) *
                              ((N + d.NWV * 16 * d.NTW - 1) / (d.NWV * 16 * d.NTW)) * (K / KBLK);
      if (units < 1024) variant = f8 ? 3 : 4;  // fp8: the 32-row tile (an even row-tile count)
    }
  }
  if (variant >= count) return -8;
  const TVariant& v = table[variant];
  if (variant_fn(v, mode) == nullptr) return -8;  // e.g. fp8 with odd row tiles
  const int BM = 16 * v.MT, BN = v.NWV * 16 * v.NTW;
  const int Gk = K / KBLK;
  TiledPlan q;
  q.variant = variant;
  q.mode = mode;
  q.args.M = M;
  q.args.N = N;
  q.args.K = K;
  q.args.tiles_m = (M + BM - 1) / BM;
  q.args.tiles_n = (N + BN - 1) / BN;
  // tiles are handed out in groups of 4 row tiles (then the next column tiles): the 32
  // workgroups of an XCD then share 4 row tiles of X and 8 column tiles of W in its L2
  // (measured 0-8% faster than groups of 8 on the 70B-class layers)
  q.args.group_m = 4;
  q.args.xscale = nullptr;
  q.args.out_bf16 = mode_bf16(mode) ? 1 : 0;
  const long T = (long)q.args.tiles_m * q.args.tiles_n;
  if (T > (1L << 30)) return -2;
  // buffer offsets are 32-bit: the rows of X and Y one tile touches, and the fp16
  // weight rows of one wave, must stay below 2 GiB from their base
  const long long xrows = BM > 16 * v.NTW ? BM : 16 * v.NTW;
  if (xrows * K * 2 >= (1LL << 31) || (long long)BM * N * 2 >= (1LL << 31)) return -2;
  if (grid <= 0) {
    // one workgroup per compute unit; fewer for small problems, so that a stripe
    // holds at least a few k-blocks
    const long min_units = 8;
    long g = (T * Gk + min_units - 1) / min_units;
    grid = (int)(g < 256 ? (g < 1 ? 1 : g) : 256);
    // the eight-wave tiles: whole rounds of 224-256 workgroups where the tile count allows
    // (their stream-K pieces cost about half a tile's work per workgroup)
    if (v.NWV == 8 && dp_grid(T) > 0) grid = (int)dp_grid(T);
    // 200-255 tiles: one workgroup per tile, whole K, no stream-K pieces (measured 1.02x
    // at M = 256 on 8192 x 28672 with 224 tiles, 1.07x at M = 128 on 8192 x 28672 with
    // 128 x 128 tiles, 1.12x at M = 256 on 5120 x 13824 with 216 tiles)
    if (T >= 200 && T < 256 && grid == 256) grid = (int)T;
    // fewer tiles than that: k = 256 / T workgroups per tile when they cut every tile into
    // k equal whole-k-block pieces and still fill 200-256 compute units (1.04-1.10x for the
    // zero-point layers of 5120 x 13824 and 13824 x 5120 at M = 48 / 128, 1.06x for the
    // 2:4 32-row tiles and 1.04x at M = 128 on 8192 x 28672; with fp8 activations 0.95x)
    if (T < 200 && grid == 256 && mode != W_SYM8 && mode != W_ASYM8) {
      const long k = 256 / T;
      if (T * k >= 200 && Gk % k == 0) grid = (int)(T * k);
    }
    // short K (at most 32 k-blocks) on the four-wave 128 x 128 tiles with fp16 activations
    // (or rows rewritten in fp16): whole pieces even when they fill only 160-199 compute
    // units, since a stream-K stripe's fixed cost weighs more against so short a tile
    // (1.02-1.09x at M = 128 / 256 on 4096 x 11008 and 4096 x 12288)
    if (T < 200 && grid == 256 && Gk <= 32 && v.MT == 8 && v.NTW == 2 && v.NWV == 4 &&
        (mode == W_SYM || mode == W_ASYM || mode == W_SYM64 || mode == W_ASYM64)) {
      const long k = 256 / T;
      if (T * k >= 160 && Gk % k == 0) grid = (int)(T * k);
    }
  }
  if ((long long)grid > (long long)T * Gk) grid = (int)(T * Gk);  // at least one unit each
  q.args.grid = grid;
  // four-wave tiles: all but the last one or two rounds of tiles are data-parallel, the
  // rest (between one and two rounds' worth) is striped; striping only the remainder
  // (shorter stripes, all ending together) was 3-5% slower on the 70B shapes.  Eight-wave
  // tiles: every full round is data-parallel and only the remainder is striped, which
  // halves the fp32 pieces their larger tiles write and the second pass reads (measured
  // 1.05x at M = 1024 and 1.04x at M = 4096 on 8192 x 10240, 1.02x at M = 1024 on
  // 5120 x 13824, within 1% elsewhere).
  const long full = T / grid;
  long dp_tiles;
  if (T % grid == 0) dp_tiles = T;
  else if (full >= 1) dp_tiles = (v.NWV == 8 ? full : full - 1) * grid;
  else dp_tiles = 0;
  q.args.dp_rounds = (int)(dp_tiles / grid);
  const long sk_tiles = T - dp_tiles;
  q.args.sk_units = (long long)sk_tiles * Gk;
  q.args.sk_per_wg = (q.args.sk_units + grid - 1) / grid;
  if (q.args.sk_per_wg < 1) q.args.sk_per_wg = 1;
  // the kernel keeps its stripe bookkeeping in 32 bits
  if (q.args.sk_units + q.args.sk_per_wg + Gk >= (1LL << 31)) return -2;
  if ((long long)sk_tiles * v.MT > (1LL << 30)) return -2;
  q.fixup_wgs = (int)sk_tiles * v.MT;  // one workgroup per (stream-K tile, row tile)
  q.part_floats = sk_tiles ? (size_t)2 * grid * BM * BN : 0;
  q.wgs = grid;
  q.threads = 64 * v.NWV;
  *p = q;
  return 0;
}

hipError_t tiled_launch(const TiledPlan& p, const uint16_t* X, const void* w, const uint16_t* sp,
                        const uint32_t* zp, uint16_t* Y, float* part, hipStream_t st,
                        const float* xscale, bool rows16, bool bf16_out) {
  const TVariant& v = p.mode == W_FP16 ? kTiledF16[p.variant] : kTiled[p.variant];
  TiledFn fn = variant_fn(v, p.mode);
  if (fn == nullptr) return hipErrorInvalidValue;  // not reachable through tiled_make_plan
  if ((rows16 || bf16_out) && (mode_fp8(p.mode) || mode_bf16(p.mode) || p.mode == W_SP24 ||
                               p.mode == W_FP16))
    return hipErrorInvalidValue;
  TiledArgs args = p.args;
  args.xscale = mode_fp8(p.mode) || rows16 ? xscale : nullptr;
  if (bf16_out) args.out_bf16 = 1;
  hipLaunchKernelGGL(fn, dim3(p.wgs), dim3(p.threads), 0, st, X,
                     reinterpret_cast<const uint32_t*>(w), sp, zp, Y, part, args);
  if (p.fixup_wgs > 0) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(v.fixup, dim3(p.fixup_wgs), dim3(p.threads), 0, st, part, Y, args);
  }
  return hipGetLastError();
}

}  // namespace w4a16
