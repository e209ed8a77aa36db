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
//   * One wave owns NT tiles of 16 columns and the XR-row block of X (XR = 4, 8,
//     16, 32 or 64; MT = ceil(XR/16) MFMA row tiles).  A 128-row k-block of one
//     tile is 1 KiB of packed codes in the repacked layout: one 16-byte
//     non-temporal buffer load per lane (layout in internal.h).
//   * Activations are loaded as whole rows (each instruction covers 4 rows x 256
//     bytes, lanes past M read zeros through the buffer bounds) and re-laid into
//     MFMA fragments through a wave-private LDS tile.  Loading the fragments
//     straight from memory touches 16 rows x 64 bytes per instruction and was
//     measured 2.6x slower from L2 on MI355X than the row-contiguous pattern.
//   * Dequantization uses the 0x6400 exponent trick: OR-ing a nibble into the
//     mantissa of 1024.0 gives the exact fp16 1024+q (or 1024+16q for the high
//     nibble of a byte), and one packed fp16 add / fma removes the offset and the
//     zero-point, giving the exact integer q - z.  With one or two column tiles per
//     wave the scale is applied after the four v_mfma_f32_16x16x32_f16 of the
//     k-block, in fp32, on the 4 accumulators of the lane (1 fma per output instead
//     of 1 multiply per weight); with three or more, the weights are multiplied by
//     the scale in fp16 (one rounding, as in the dequantized fp16 weight) and the
//     matrix instructions accumulate straight into the output registers.
//   * The WK waves of a workgroup take interleaved k-blocks of the K range of the
//     same output tiles and reduce through LDS in a fixed order.
//   * When a tile's K range is cut into `splits` slices owned by different
//     workgroups, each writes an fp32 partial, bumps an arrival counter, and the
//     last to arrive sums the slices in slice order (deterministic) and writes
//     Y; it also resets the counter for the next launch, so no memset is needed.
//   * Each wave keeps D k-blocks of loads in flight in a register ring; the loop
//     is branch-free so that the compiler's wait counts stay exact.
#include "internal.h"

namespace w4a16 {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half16 __attribute__((ext_vector_type(16)));

// Buffer resources: the uniform part of an address goes to the scalar offset, the
// per-lane part to a fixed VGPR offset, and lanes whose offset is past num_records
// read zeros without touching memory (used for rows of X beyond M), so no branch
// is needed around any load.  Word 3 (0x00020000) is the gfx9-family raw-buffer
// format.  Each resource covers one workgroup's region, so offsets stay small.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                          0x00020000);
}
template <bool STREAM>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4,
                            __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, STREAM ? 2 : 0));
}


// (w & mask) | magic in one VALU op.  The compiler otherwise emits an and and an
// or, because gfx9 VOP3 can read only one scalar/literal operand: keep the mask
// in an SGPR and the magic number in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

// 8 codes of one repacked word -> 8 exact fp16 (q - z), in row order 0..7.
// c0 = -(1024 + z) and c1 = -(64 + z) in both halves.
__device__ __forceinline__ half8 dequant_word(uint32_t w, half2v c0, half2v c1, uint32_t magic) {
  const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w8 = w >> 8;
  const uint32_t t0 = and_or(w, 0x000F000Fu, magic);   // 1024+q0 | 1024+q1
  const uint32_t t1 = and_or(w, 0x00F000F0u, magic);   // 1024+16q2 | 1024+16q3
  const uint32_t t2 = and_or(w8, 0x000F000Fu, magic);  // 1024+q4 | 1024+q5
  const uint32_t t3 = and_or(w8, 0x00F000F0u, magic);  // 1024+16q6 | 1024+16q7
  const half2v h0 = __builtin_bit_cast(half2v, t0) + c0;
  const half2v h1 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, t1), sixteenth, c1);
  const half2v h2 = __builtin_bit_cast(half2v, t2) + c0;
  const half2v h3 = __builtin_elementwise_fma(__builtin_bit_cast(half2v, t3), sixteenth, c1);
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 activations: 8 codes of one repacked word -> 8 exact bf16 values 128 + q, rows
// 0..7.  OR-ing a nibble into the mantissa of 128.0 (0x4300; the bf16 ulp in [128, 256)
// is 1) gives 128 + q exactly; the shifts bring each row pair's nibbles to bits 0-3 of
// the two halves (bf16 has only 7 mantissa bits, so the 16q trick of fp16 does not
// apply).  The offset 128 + z is removed after the matrix instruction, in fp32, with
// the block's activation row sums (see compute_stage).
// These words go straight into a matrix instruction, so they are formed in plain code
// rather than with the and_or asm above: the compiler inserts the wait states a matrix
// instruction needs after a VALU write of its operands only for instructions it knows
// (a bf16 kernel whose schedule put the asm right before the matrix instruction read
// stale operands on MI355X).
__device__ __forceinline__ bf16x8 offset_codes_bf16(uint32_t w) {
  const uint32_t magic = 0x43004300u;
  const uint32_t t0 = (w & 0x000F000Fu) | magic;          // rows 0, 1
  const uint32_t t1 = ((w >> 4) & 0x000F000Fu) | magic;   // rows 2, 3
  const uint32_t t2 = ((w >> 8) & 0x000F000Fu) | magic;   // rows 4, 5
  const uint32_t t3 = ((w >> 12) & 0x000F000Fu) | magic;  // rows 6, 7
  typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(bf16x8, u32x4v{t0, t1, t2, t3});
}

typedef short short2v __attribute__((ext_vector_type(2)));

// fp8 activations: 8 codes of one repacked word -> 8 OCP E4M3 bytes of the exact integer
// q - z, rows 0..7 in bytes 0..7 (the operand of one v_mfma_f32_16x16x32_fp8_fp8).  The
// integers come out of dequant_word exactly in fp16; every integer in [-15, 15] is exact
// in E4M3 (3 mantissa bits cover integers up to 16), so the conversion, a unit-scale
// v_cvt_scalef32_pk_fp8_f16 per pair, is exact too.
__device__ __forceinline__ uint64_t dequant_word_fp8(uint32_t w, half2v c0, half2v c1,
                                                     uint32_t magic) {
  const half8 h = dequant_word(w, c0, c1, magic);
  short2v lo = {0, 0}, hi = {0, 0};
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(lo, half2v{h[0], h[1]}, 1.0f, false);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(lo, half2v{h[2], h[3]}, 1.0f, true);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(hi, half2v{h[4], h[5]}, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(hi, half2v{h[6], h[7]}, 1.0f, true);
  return (uint64_t)__builtin_bit_cast(uint32_t, lo) |
         ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32);
}

// fp32 -> output bits: fp16 (round to nearest even), or bf16 (round to nearest even)
template <int MODE>
__device__ __forceinline__ uint16_t out_bits(float v) {
  if constexpr (mode_bf16(MODE)) {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  } else {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
  }
}

// bytes per X row in the LDS tile.  fp16 / bf16: 256 + 32, the smallest padding whose
// 16-byte fragment reads (16 rows, one column of chunks) are free of bank conflicts on
// gfx950 (counted with SQ_LDS_BANK_CONFLICT: 256 + 16, + 48 and + 64 conflict, + 32 reads
// 0).  fp8 rows (128 bytes used): 256 + 16, which gives its 8-byte fragment reads a third
// of the conflicts that 256 + 32 does.
template <int MODE>
__host__ __device__ constexpr int x_stride() {
  return mode_fp8(MODE) ? 272 : 288;
}

// 16-byte activation loads per k-block: one covers 4 rows x 256 bytes of fp16 / bf16, or
// 8 rows x 128 bytes of fp8
__host__ __device__ constexpr int x_loads(int XR, int MODE) {
  return mode_fp8(MODE) ? (XR + 7) / 8 : XR / 4;
}
__host__ __device__ constexpr int x_elem_bytes(int MODE) { return mode_fp8(MODE) ? 1 : 2; }


template <int XR, int NT, int MODE>
struct Stage {
  u32x4 w[NT][MODE == W_FP16 ? 4 : 1];  // packed codes (fp16 rows for the baseline; for 2:4,
                                        // .x/.y = kept codes of the two halves, .z = positions)
  uint16_t s[NT];                       // fp16 scale bits of the lane's column
  uint2 z[NT];                          // 16 zero-points of the tile (ASYM)
  uint32_t s64[NT];                     // groups of 64: the scales of both halves (low: rows 0-63)
  u32x4 z64[NT];                        // groups of 64: zero-points, .xy half 0, .zw half 1
  uint2 s4[NT];                         // 2:4: the four scales of the lane's four columns
  u32x4 x[x_loads(XR, MODE)];           // X rows 4c + lane/16, 16-byte chunk lane%16 (fp8:
                                        // rows 8c + lane/8, chunk lane%8)
};

// Loads of one k-block.  kb is wave-uniform, so every scalar offset below is
// formed on the scalar unit; the per-lane offsets were computed once.
struct Rsrc {
  rsrc_t w, s, z, x;
  uint32_t lane_w;  // byte offset of the lane inside a weight block (or fp16 row slice)
};

// `live` is wave-uniform: past the wave's last k-block every load goes through a
// resource of zero size, which returns zeros without a memory request, so the
// pipelined loop below needs no branch (branches would make the compiler's wait
// counts conservative and serialize the prefetch).
template <int XR, int NT, int MODE>
__device__ __forceinline__ void load_stage(Stage<XR, NT, MODE>& S, int kb, bool live, int lane,
                                           int Gk, int K, const Rsrc& R0, const Rsrc& Rnull,
                                           const uint32_t xoff[x_loads(XR, MODE)]) {
  const Rsrc& R = live ? R0 : Rnull;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (MODE == W_FP16) {
      // baseline: W is fp16 [N][K]; the lane's column, rows 32j + 8(lane/16) + 0..7
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S.w[t][j] = bload16<true>(R.w, R.lane_w + (uint32_t)(t * 16 * K * 2 + 64 * j),
                                  (uint32_t)kb * KBLK * 2);
    } else if (MODE == W_SP24) {
      const uint32_t blk = (uint32_t)(t * Gk + kb);
      const uint2 c = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(R.w, R.lane_w, blk * 512u, 2));
      S.w[t][0].x = c.x;
      S.w[t][0].y = c.y;
      S.w[t][0].z = __builtin_amdgcn_raw_buffer_load_b32(R.z, (uint32_t)lane * 4, blk * 256u, 2);
      S.s4[t] = __builtin_bit_cast(
          uint2, __builtin_amdgcn_raw_buffer_load_b64(R.s, (uint32_t)(lane >> 4) * 8, blk * 32u, 0));
    } else {
      const uint32_t blk = (uint32_t)(t * Gk + kb);
      S.w[t][0] = bload16<true>(R.w, R.lane_w, blk * 1024u);
      if constexpr (mode_g64(MODE)) {
        S.s64[t] = __builtin_amdgcn_raw_buffer_load_b32(R.s, (uint32_t)(lane & 15) * 4, blk * 64u, 0);
        if (mode_asym(MODE))
          S.z64[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(R.z, 0u, blk * 16u, 0));
      } else {
        S.s[t] = __builtin_amdgcn_raw_buffer_load_b16(R.s, (uint32_t)(lane & 15) * 2, blk * 32u, 0);
        if (mode_asym(MODE))
          S.z[t] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(R.z, 0u, blk * 8u, 0));
      }
    }
  }
#pragma unroll
  for (int c = 0; c < x_loads(XR, MODE); ++c)
    S.x[c] = bload16<false>(R.x, xoff[c], (uint32_t)kb * KBLK * x_elem_bytes(MODE));
}

// The lane's column's zero-point code (8 when symmetric) and fp32 scale for half h of
// column tile t (h = 0 unless the groups are 64 rows: then words j = 2h, 2h + 1 of the
// block belong to half h).
template <int XR, int NT, int MODE>
__device__ __forceinline__ int zero_code(const Stage<XR, NT, MODE>& S, int t, int h, int lane) {
  if constexpr (!mode_asym(MODE)) {
    return 8;
  } else {
    const int c = lane & 15;
    uint32_t zw;
    if constexpr (mode_g64(MODE))
      zw = h == 0 ? (c < 8 ? S.z64[t].x : S.z64[t].y) : (c < 8 ? S.z64[t].z : S.z64[t].w);
    else
      zw = c < 8 ? S.z[t].x : S.z[t].y;
    return (int)((zw >> (4 * (c & 7))) & 15u);
  }
}
template <int XR, int NT, int MODE>
__device__ __forceinline__ float block_scale(const Stage<XR, NT, MODE>& S, int t, int h) {
  if constexpr (mode_g64(MODE))
    return (float)__builtin_bit_cast(half2v, S.s64[t])[h];
  else
    return (float)__builtin_bit_cast(_Float16, S.s[t]);
}

// Compute one k-block: lay the X rows into the wave's LDS tile, read them back as
// MFMA fragments (lane l: row 16mt + l%16, 8 halves at 32j + 8(l/16)), dequantize
// the codes and run the four MFMAs per (row tile, column tile).
template <int XR, int NT, int MODE>
__device__ __forceinline__ void compute_stage(const Stage<XR, NT, MODE>& S,
                                              float4v (&acc)[NT][(XR + 15) / 16], int lane,
                                              uint32_t magic, char* xlds) {
  constexpr int MT = (XR + 15) / 16;
  if constexpr (mode_fp8(MODE)) {
    // fp8 activations: rows of 128 bytes; fragment (mt, j) of lane l is the 8 bytes of row
    // 16mt + l%16 at 32j + 8(l/16), the k-slots of the word j of the lane's weight block.
    // The weights enter v_mfma_f32_16x16x32_fp8_fp8 as the exact integers q - z and the
    // scale applies in fp32 per block, for any number of column tiles.
#pragma unroll
    for (int c = 0; c < x_loads(XR, MODE); ++c)
      *reinterpret_cast<u32x4*>(xlds + (8 * c + (lane >> 3)) * x_stride<MODE>() + (lane & 7) * 16) = S.x[c];
    long a8[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        a8[mt][j] = *reinterpret_cast<const long*>(xlds + (mt * 16 + (lane & 15)) * x_stride<MODE>() +
                                                    32 * j + 8 * (lane >> 4));
    constexpr int SH = mode_g64(MODE) ? 2 : 1;  // scale / zero-point halves per block
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      half2v c0[SH], c1[SH];
      float sc[SH];
#pragma unroll
      for (int h = 0; h < SH; ++h) {
        const int zq = zero_code(S, t, h, lane);
        const _Float16 a0 = (_Float16)(float)(-1024 - zq);
        const _Float16 a1 = (_Float16)(float)(-64 - zq);
        c0[h] = half2v{a0, a0};
        c1[h] = half2v{a1, a1};
        sc[h] = block_scale(S, t, h);
      }
      long b[4];
      b[0] = (long)dequant_word_fp8(S.w[t][0].x, c0[0], c1[0], magic);
      b[1] = (long)dequant_word_fp8(S.w[t][0].y, c0[0], c1[0], magic);
      b[2] = (long)dequant_word_fp8(S.w[t][0].z, c0[SH - 1], c1[SH - 1], magic);
      b[3] = (long)dequant_word_fp8(S.w[t][0].w, c0[SH - 1], c1[SH - 1], magic);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // one fp32 partial per half (k-steps 0-1 and 2-3), each with its group's scale
        float4v g[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          g[SH == 2 ? j >> 1 : 0] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(
              a8[mt][j], b[j], g[SH == 2 ? j >> 1 : 0], 0, 0, 0);
        acc[t][mt] += sc[0] * g[0];
        if constexpr (SH == 2) acc[t][mt] += sc[1] * g[1];
      }
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < XR / 4; ++c)
    *reinterpret_cast<u32x4*>(xlds + (4 * c + (lane >> 4)) * x_stride<MODE>() + (lane & 15) * 16) = S.x[c];
  half8 a[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      a[mt][j] = *reinterpret_cast<const half8*>(xlds + (mt * 16 + (lane & 15)) * x_stride<MODE>() +
                                                  64 * j + 16 * (lane >> 4));
  if (MODE == W_SP24) {
    // 2:4: W is the sparse A operand (lane: column 4(l/16)+r ... see the epilogue), X the
    // dense B operand: its 16 halves for half h are the fragments 2h and 2h+1 above.
    const half2v c0 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const half2v c1 = {(_Float16)-72.0f, (_Float16)-72.0f};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const half8 w0 = dequant_word(S.w[t][0].x, c0, c1, magic);
      const half8 w1 = dequant_word(S.w[t][0].y, c0, c1, magic);
      const int meta = (int)S.w[t][0].z;
      const half2v s01 = __builtin_bit_cast(half2v, S.s4[t].x);
      const half2v s23 = __builtin_bit_cast(half2v, S.s4[t].y);
      const float4v sc = {(float)s01[0], (float)s01[1], (float)s23[0], (float)s23[1]};
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const half16 xb0 = __builtin_shufflevector(a[mt][0], a[mt][1], 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                                   9, 10, 11, 12, 13, 14, 15);
        const half16 xb1 = __builtin_shufflevector(a[mt][2], a[mt][3], 0, 1, 2, 3, 4, 5, 6, 7, 8,
                                                   9, 10, 11, 12, 13, 14, 15);
        float4v g = {0.f, 0.f, 0.f, 0.f};
        g = __builtin_amdgcn_smfmac_f32_16x16x64_f16(w0, xb0, g, meta, 0, 0);
        g = __builtin_amdgcn_smfmac_f32_16x16x64_f16(w1, xb1, g, meta, 0, 1);
        acc[t][mt] += sc * g;
      }
    }
    return;
  }
  if constexpr (mode_bf16(MODE)) {
    // bf16: the matrix instructions see the exact 128 + q; per (row tile, block) the
    // sum of the activations over the block (one more matrix instruction per k-step
    // against ones) removes the offset: sum x (q - z) = sum x (128 + q) - (128 + z) sum x.
    // The weights stay exact integers and the scale applies in fp32, as in the fp16 path.
    // With groups of 64 rows, everything is kept per half of the block (k-steps 0-1 and
    // 2-3): activation sums, partial products, offsets and scales.
    constexpr int SH = mode_g64(MODE) ? 2 : 1;
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                         0x3F803F80u});
    float4v xs[MT][SH];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int h = 0; h < SH; ++h) xs[mt][h] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xs[mt][SH == 2 ? j >> 1 : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a[mt][j]), ones, xs[mt][SH == 2 ? j >> 1 : 0], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf16x8 b[4];
      b[0] = offset_codes_bf16(S.w[t][0].x);
      b[1] = offset_codes_bf16(S.w[t][0].y);
      b[2] = offset_codes_bf16(S.w[t][0].z);
      b[3] = offset_codes_bf16(S.w[t][0].w);
      float off[SH], sc[SH];
#pragma unroll
      for (int h = 0; h < SH; ++h) {
        off[h] = (float)(128 + zero_code(S, t, h, lane));
        sc[h] = block_scale(S, t, h);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float4v g[SH];
#pragma unroll
        for (int h = 0; h < SH; ++h) g[h] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          g[SH == 2 ? j >> 1 : 0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, a[mt][j]), b[j], g[SH == 2 ? j >> 1 : 0], 0, 0, 0);
#pragma unroll
        for (int h = 0; h < SH; ++h) acc[t][mt] += sc[h] * (g[h] - off[h] * xs[mt][h]);
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    half8 b[4];
    if (MODE == W_FP16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = __builtin_bit_cast(half8, S.w[t][j]);
    } else {
      // the offsets -(1024 + z), -(64 + z) of each half (both halves alike unless the
      // groups are 64 rows): words j = 0, 1 are rows 0-63 of the block, j = 2, 3 rows 64-127
      constexpr int SH = mode_g64(MODE) ? 2 : 1;
      half2v c0[SH], c1[SH];
#pragma unroll
      for (int h = 0; h < SH; ++h) {
        int zq = 8;
        if constexpr (mode_asym(MODE)) {
          const int c = lane & 15;
          uint32_t zw;
          if constexpr (SH == 2) zw = h == 0 ? (c < 8 ? S.z64[t].x : S.z64[t].y)
                                             : (c < 8 ? S.z64[t].z : S.z64[t].w);
          else zw = c < 8 ? S.z[t].x : S.z[t].y;
          zq = (int)((zw >> (4 * (c & 7))) & 15u);
        }
        const _Float16 a0 = (_Float16)(float)(-1024 - zq);
        const _Float16 a1 = (_Float16)(float)(-64 - zq);
        c0[h] = half2v{a0, a0};
        c1[h] = half2v{a1, a1};
      }
      b[0] = dequant_word(S.w[t][0].x, c0[0], c1[0], magic);
      b[1] = dequant_word(S.w[t][0].y, c0[0], c1[0], magic);
      b[2] = dequant_word(S.w[t][0].z, c0[SH - 1], c1[SH - 1], magic);
      b[3] = dequant_word(S.w[t][0].w, c0[SH - 1], c1[SH - 1], magic);
    }
    if constexpr (NT >= 3 && MODE != W_FP16) {
      // many column tiles per wave: multiply the weights by the scale in fp16 (one
      // rounding of W, the fp16 dequantized weight) and accumulate straight into acc;
      // measured faster than rescaling the fp32 partial sum of every (tile, row tile)
      _Float16 sh0, sh1;
      if constexpr (mode_g64(MODE)) {
        const half2v s01 = __builtin_bit_cast(half2v, S.s64[t]);
        sh0 = s01[0];
        sh1 = s01[1];
      } else {
        sh0 = sh1 = __builtin_bit_cast(_Float16, S.s[t]);
      }
      const half8 s8a = {sh0, sh0, sh0, sh0, sh0, sh0, sh0, sh0};
      const half8 s8b = {sh1, sh1, sh1, sh1, sh1, sh1, sh1, sh1};
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = b[j] * (j < 2 ? s8a : s8b);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][j], b[j], acc[t][mt], 0, 0, 0);
      continue;
    }
    // row tiles past M hold zero activations and add exactly zero; no branch here
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (MODE == W_FP16) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][j], b[j], acc[t][mt], 0, 0, 0);
      } else if constexpr (mode_g64(MODE)) {
        // one fp32 partial per 64-row half, each rescaled by its own group's scale
        float4v g0 = {0.f, 0.f, 0.f, 0.f}, g1 = {0.f, 0.f, 0.f, 0.f};
        g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][0], b[0], g0, 0, 0, 0);
        g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][1], b[1], g0, 0, 0, 0);
        g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][2], b[2], g1, 0, 0, 0);
        g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][3], b[3], g1, 0, 0, 0);
        const half2v s01 = __builtin_bit_cast(half2v, S.s64[t]);
        acc[t][mt] += (float)s01[0] * g0 + (float)s01[1] * g1;
      } else {
        // two accumulation chains of two matrix instructions each (the k-steps j = 0, 2
        // and 1, 3): half the dependent latency of one chain of four
        const float4v z = {0.f, 0.f, 0.f, 0.f};
        float4v g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][0], b[0], z, 0, 0, 0);
        float4v g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][1], b[1], z, 0, 0, 0);
        g0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][2], b[2], g0, 0, 0, 0);
        g1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][3], b[3], g1, 0, 0, 0);
        const float sc = (float)__builtin_bit_cast(_Float16, S.s[t]);
        acc[t][mt] += sc * (g0 + g1);
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

template <int XR, int NT, int WK, int D, int MODE>
__global__ __launch_bounds__(64 * WK) void skinny_kernel(
    const uint16_t* __restrict__ X, const uint4* __restrict__ W, const uint16_t* __restrict__ Sp,
    const uint2* __restrict__ Zp, uint16_t* __restrict__ Y, float* __restrict__ part,
    int* __restrict__ counters, int M, int N, int K, int splits, int nblocks,
    const float* __restrict__ xscale) {
  constexpr int MT = (XR + 15) / 16;
  constexpr int XTILE = MT * 16 * x_stride<MODE>();  // bytes of one wave's X tile
  // per-wave X tiles; after the main loop the same memory holds the reduction (which
  // needs more than the tiles for eight column tiles per wave)
  constexpr int RED = (WK - 1) * 64 * NT * MT * 16;
  constexpr int LDSB = RED > WK * XTILE ? RED : WK * XTILE;
  __shared__ __attribute__((aligned(16))) char lds[LDSB];
  const int lane = threadIdx.x & 63;
  // wave index made uniform so that all k-block bookkeeping stays on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // workgroup -> (row block, column tiles, K slice).  The loads wait for this, so the
  // common plans (one K slice, one row block) skip the divisions; Gk * splits < 2^31
  // (the plan refuses more), so the slice bounds need no 64-bit division.
  int bid = blockIdx.x;
  const int Gk = K / KBLK;
  int sl = 0, kb0 = 0, kb1 = Gk;
  if (splits > 1) {
    sl = bid % splits;
    bid /= splits;
    kb0 = Gk * sl / splits;
    kb1 = Gk * (sl + 1) / splits;
  }
  int nb = bid, mb = 0;
  if (bid >= nblocks) {
    nb = bid % nblocks;
    mb = bid / nblocks;
  }
  // K range of this workgroup's slice, then this wave's k-blocks in it
  const int nk_wg = kb1 - kb0;
  // wave w takes the k-blocks kb0 + w, kb0 + w + WK, ...: the waves of a workgroup read
  // neighbouring 1 KiB blocks at the same time (measured 1-6% faster on the decode
  // shapes than contiguous chunks per wave)
  const int kw0 = kb0 + wave;
  const int nk = nk_wg > wave ? (nk_wg - wave + WK - 1) / WK : 0;
  const int t0 = nb * NT;
  const int m0 = mb * XR;
  char* xlds = lds + wave * XTILE;

  // buffer resources over this workgroup's tiles and rows
  Rsrc R;
  if (MODE == W_FP16) {
    const char* wbase = reinterpret_cast<const char*>(W) + (size_t)t0 * 16 * K * 2;
    R.w = make_rsrc(wbase, (uint32_t)(NT * 16 * K * 2));
    R.lane_w = (uint32_t)(((lane & 15) * K + 8 * (lane >> 4)) * 2);
  } else if (MODE == W_SP24) {
    // kept codes (512 B per block), positions (256 B per block, passed as Zp), scales
    R.w = make_rsrc(reinterpret_cast<const char*>(W) + (size_t)t0 * Gk * 512,
                    (uint32_t)(NT * Gk * 512));
    R.z = make_rsrc(reinterpret_cast<const char*>(Zp) + (size_t)t0 * Gk * 256,
                    (uint32_t)(NT * Gk * 256));
    R.s = make_rsrc(Sp + (size_t)t0 * Gk * 16, (uint32_t)(NT * Gk * 32));
    R.lane_w = (uint32_t)lane * 8;
  } else {
    constexpr int SH = mode_g64(MODE) ? 2 : 1;  // scale / zero-point rows per block
    R.w = make_rsrc(reinterpret_cast<const char*>(W) + (size_t)t0 * Gk * 1024,
                    (uint32_t)(NT * Gk * 1024));
    R.s = make_rsrc(Sp + (size_t)t0 * Gk * 16 * SH, (uint32_t)(NT * Gk * 32 * SH));
    if (mode_asym(MODE)) R.z = make_rsrc(Zp + (size_t)t0 * Gk * SH, (uint32_t)(NT * Gk * 8 * SH));
    R.lane_w = (uint32_t)lane * 16;
  }
  const int rows = M - m0 < XR ? M - m0 : XR;  // valid rows of this block of X
  constexpr int XB = x_elem_bytes(MODE);
  R.x = make_rsrc(reinterpret_cast<const char*>(X) + (size_t)m0 * K * XB, (uint32_t)(rows * K * XB));
  // per-lane byte offsets of the X row loads: row 4c + lane/16, 16 bytes at byte
  // 16(lane%16) of the row's k-block (fp8: row 8c + lane/8, byte 16(lane%8)); rows past M
  // read zeros
  uint32_t xoff[x_loads(XR, MODE)];
#pragma unroll
  for (int c = 0; c < x_loads(XR, MODE); ++c) {
    const int r = mode_fp8(MODE) ? 8 * c + (lane >> 3) : 4 * c + (lane >> 4);
    const int cb = mode_fp8(MODE) ? 16 * (lane & 7) : 16 * (lane & 15);
    xoff[c] = r < rows ? (uint32_t)(r * K * XB + cb) : kOutOfRange;
  }
  const uint32_t magic = 0x64006400u;

  float4v acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = float4v{0.f, 0.f, 0.f, 0.f};

  // a resource of zero size: loads through it return zeros and touch no memory
  Rsrc Rnull;
  Rnull.w = make_rsrc(W, 0);
  Rnull.s = make_rsrc(Sp, 0);
  Rnull.z = make_rsrc(Zp, 0);
  Rnull.x = make_rsrc(X, 0);
  Rnull.lane_w = R.lane_w;

  // register ring of D stages: D k-blocks in flight ahead of the one being computed.
  // The trip count is rounded up to a multiple of D; stages past the wave's range
  // hold zeros and add exactly zero.
  Stage<XR, NT, MODE> S[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_stage(S[d], kw0 + d * WK, d < nk, lane, Gk, K, R, Rnull, xoff);
    __builtin_amdgcn_sched_barrier(0);  // issue the stages in order
  }
  // rows XR..15 of the LDS tile are never written by the loads: keep them zero (after
  // the first loads are on their way)
  if (XR % 16 != 0) {
    for (int i = lane; i < (16 - XR) * x_stride<MODE>() / 16; i += 64)
      *reinterpret_cast<u32x4*>(xlds + XR * x_stride<MODE>() + 16 * i) = u32x4{0, 0, 0, 0};
  }
  for (int i = 0; i < nk; i += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      compute_stage(S[d], acc, lane, magic, xlds);
      load_stage(S[d], kw0 + (i + d + D) * WK, i + d + D < nk, lane, Gk, K, R, Rnull, xoff);
      // keep stage order: the compiler would otherwise merge the stages and wait
      // for every outstanding load before the first one is computed
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- in-workgroup reduction over the WK waves, fixed order 0, 1, ..., WK-1 ----
  // (reuses the X tiles: wait until every wave is done with its tile)
  constexpr int NACC = NT * MT * 4;
  if (WK > 1) {
    // [wave-1][t][mt][lane]: the 64 lanes of one access write or read 1 KiB in a row,
    // which spreads them over every bank (a [lane][t][mt] order puts the lanes NT*MT*16
    // bytes apart: an 8-way bank conflict for NT*MT = 8)
    float4v* red = reinterpret_cast<float4v*>(lds);
    __syncthreads();
    if (wave > 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) red[(((wave - 1) * NT + t) * MT + mt) * 64 + lane] = acc[t][mt];
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WK; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] += red[(((w - 1) * NT + t) * MT + mt) * 64 + lane];
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
    // slice by slice, in slice order; the NACC loads of a slice are independent and go
    // out together, so the hand-off costs one memory round trip per slice (a loop over
    // slices inside each element would wait once per element and slice)
    const float* base = part + tile_id * splits * (NACC * 64);
    float sum[NACC];
#pragma unroll
    for (int i = 0; i < NACC; ++i) sum[i] = 0.f;
    for (int s2 = 0; s2 < splits; ++s2) {
      float v[NACC];
#pragma unroll
      for (int i = 0; i < NACC; ++i) v[i] = load_coherent(base + (long)s2 * (NACC * 64) + i * 64 + lane);
#pragma unroll
      for (int i = 0; i < NACC; ++i) sum[i] += v[i];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][mt][r] = sum[(t * MT + mt) * 4 + r];
    if (lane == 0)
      __hip_atomic_store(counters + tile_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+r of each m-tile, column lane%16 ----
  // (only the XR rows of this block: with XR < 16 the rest of the MFMA tile is padding)
  const int row_end = M < m0 + XR ? M : m0 + XR;
  if (MODE == W_SP24) {
    // 2:4 kernels compute Y^T: the lane holds row 16mt + lane%16 and the four
    // consecutive columns 4(lane/16) .. +3 of the tile (one 8-byte store)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int row = m0 + mt * 16 + (lane & 15);
        const int col = (t0 + t) * 16 + 4 * (lane >> 4);
        if (row < row_end) {
          uint2 v;
          v.x = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[t][mt][0]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[t][mt][1]) << 16);
          v.y = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[t][mt][2]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)acc[t][mt][3]) << 16);
          *reinterpret_cast<uint2*>(Y + (long)row * N + col) = v;
        }
      }
    return;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + mt * 16 + 4 * (lane >> 4) + r;
        const int col = (t0 + t) * 16 + (lane & 15);
        if (row < row_end) {
          float v = acc[t][mt][r];
          if (mode_fp8(MODE) && xscale != nullptr) v *= xscale[row];
          Y[(long)row * N + col] = out_bits<MODE>(v);
        }
      }
}

typedef void (*KernelFn)(const uint16_t*, const uint4*, const uint16_t*, const uint2*, uint16_t*,
                         float*, int*, int, int, int, int, int, const float*);

struct Variant {
  int XR, NT, WK, D;
  KernelFn sym, asym, f16, sp24, sym64, asym64, symb, asymb, sym8, asym8, symb64, asymb64,
      sym8g64, asym8g64;
  const char* name;
};

#define W4A16_VARIANT(XR, NT, WK, D)                                                     \
  Variant {                                                                              \
    XR, NT, WK, D, skinny_kernel<XR, NT, WK, D, W_SYM>, skinny_kernel<XR, NT, WK, D, W_ASYM>, \
        skinny_kernel<XR, NT, WK, D, W_FP16>, skinny_kernel<XR, NT, WK, D, W_SP24>,      \
        skinny_kernel<XR, NT, WK, D, W_SYM64>, skinny_kernel<XR, NT, WK, D, W_ASYM64>,   \
        skinny_kernel<XR, NT, WK, D, W_SYMB>, skinny_kernel<XR, NT, WK, D, W_ASYMB>,     \
        skinny_kernel<XR, NT, WK, D, W_SYM8>, skinny_kernel<XR, NT, WK, D, W_ASYM8>,     \
        skinny_kernel<XR, NT, WK, D, W_SYMB64>, skinny_kernel<XR, NT, WK, D, W_ASYMB64>, \
        skinny_kernel<XR, NT, WK, D, W_SYM8G64>,                                         \
        skinny_kernel<XR, NT, WK, D, W_ASYM8G64>,                                        \
        "skinny_xr" #XR "_nt" #NT "_wk" #WK "_d" #D                                      \
  }

const Variant kVariants[] = {
    W4A16_VARIANT(4, 1, 4, 4),   W4A16_VARIANT(4, 1, 8, 4),   W4A16_VARIANT(4, 2, 4, 4),
    W4A16_VARIANT(4, 1, 16, 2),  W4A16_VARIANT(8, 1, 4, 4),   W4A16_VARIANT(8, 2, 4, 4),
    W4A16_VARIANT(8, 1, 8, 4),   W4A16_VARIANT(16, 1, 4, 4),  W4A16_VARIANT(16, 2, 4, 4),
    W4A16_VARIANT(16, 1, 8, 2),  W4A16_VARIANT(16, 2, 8, 2),  W4A16_VARIANT(16, 1, 16, 2),
    W4A16_VARIANT(32, 1, 4, 2),  W4A16_VARIANT(32, 2, 4, 2),  W4A16_VARIANT(32, 1, 8, 2),
    W4A16_VARIANT(32, 2, 8, 2),  W4A16_VARIANT(64, 1, 4, 2),  W4A16_VARIANT(64, 2, 4, 2),
    W4A16_VARIANT(64, 1, 8, 2),  W4A16_VARIANT(8, 4, 4, 2),   W4A16_VARIANT(16, 4, 4, 2),
    W4A16_VARIANT(32, 4, 4, 2),  W4A16_VARIANT(16, 4, 2, 2),  W4A16_VARIANT(32, 4, 2, 2),
    W4A16_VARIANT(16, 8, 2, 2),  W4A16_VARIANT(8, 8, 2, 2),   W4A16_VARIANT(4, 2, 8, 4),
    W4A16_VARIANT(8, 2, 8, 4),   W4A16_VARIANT(8, 4, 8, 2),   W4A16_VARIANT(16, 4, 8, 2),
    W4A16_VARIANT(32, 4, 8, 2),  W4A16_VARIANT(8, 3, 4, 2),   W4A16_VARIANT(16, 3, 4, 2),
    W4A16_VARIANT(32, 3, 4, 2),  W4A16_VARIANT(4, 1, 8, 2),   W4A16_VARIANT(16, 8, 4, 2),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int find_variant(int XR, int NT, int WK, int D) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].XR == XR && kVariants[i].NT == NT && kVariants[i].WK == WK &&
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
    // Chosen from sweeps over the decode shapes on MI355X.  `wide`: enough 16-column
    // tiles to give every compute unit more than one, so a wave can take two tiles
    // and halve the activation reads per weight byte; `longk`: many 128-row blocks
    // per tile, so more waves share a tile's K range.
    const int XR = M <= 4 ? 4 : M <= 8 ? 8 : M <= 16 ? 16 : M <= 32 ? 32 : 64;
    const bool wide = N % 64 == 0 && N / 16 > 256;
    const bool longk = K / KBLK > 48;
    // From 8 rows on, wide layers give each wave several column tiles, so that the
    // activation rows a wave loads are reused over 32-64 columns: four, or three when
    // that fills the 256 compute units more evenly (N = 12288: 256 workgroups instead
    // of 192), or two when four would leave fewer than 160 workgroups (N = 5120, 8192:
    // measured 1.1-1.9x faster than four tiles with a K split across workgroups).
    int ntw = 4;
    if (wide) {
      auto fill = [](long wgs) { return (double)wgs / (256.0 * ((wgs + 255) / 256)); };
      if (N % 48 == 0 && N / 48 >= 160 && fill(N / 48) > fill(N / 64)) ntw = 3;
      if (N / (16 * ntw) < 160) ntw = 2;
    }
    const int tiles = N / 16;
    // Long K on layers with too few 64-column blocks for one per compute unit (N = 5120,
    // 8192 at K >= 12288): four column tiles per wave, four waves, and K cut into as many
    // slices as keep the workgroups within one round.  Each wave then streams its tiles
    // along half or a third of K, and the partial sums are few.  Graph-timed over 600
    // calls: 1.08-1.28x faster than two tiles per wave over the whole K at 16-32 rows on
    // 28672 x 8192 and 13824 x 5120, and at 8 rows (or on fp16 weights) where two tiles
    // per wave leave compute units idle (N = 5120: 1.10x, fp16 1.31x); where they fill the
    // chip (N = 8192) the unsplit plan is 4% (8 rows) and 11% (fp16) faster.  At K = 8192
    // two tiles still win.
    const bool fills2 = N / 32 >= 256;
    const bool longk_split = wide && ntw == 2 && XR >= 8 && XR <= 32 && K / KBLK >= 96 &&
                             (!fills2 || (XR >= 16 && mode != W_FP16));
    // fp8 activations at 5-32 rows (16-32 rows only on layers under 1024 column tiles):
    // one column tile per wave.  They rescale every (column tile, row tile) partial in fp32 per k-block, so
    // several tiles per wave only lengthen a wave's chain, and their 1-byte activations
    // leave little to share (graph-timed 1.06-1.47x faster than three or four tiles per
    // wave at M = 8-32 on 4096 x 12288, 4096 x 11008 and 8192 x 10240, and 1.02-1.18x at
    // M = 8-16 than the long-K split on 13824 x 5120; one 32-row block 1.02-1.03x
    // faster than two 16-row blocks on 4096 x 4096 and 11008 x 4096; 1.12x at M = 8 on
    // 8192 x 28672).  Above 8 rows the 1792 tiles of 8192 x 28672 keep four tiles per wave
    // (0.88-0.98x with one at M = 16-32), 32 rows keep the long-K split (0.93-0.96x with
    // one tile), and layers of 8192 columns keep their two tiles per wave (0.88-0.99x with
    // one at M = 8-32 on 8192 x 8192 and 28672 x 8192).
    const bool fp8_one = mode_fp8(mode) && XR >= 8 && XR <= 32 && (tiles < 1024 || XR == 8) &&
                         !(XR == 32 && longk_split) && !(wide && ntw == 2 && fills2);
    const bool longsplit = longk_split && !fp8_one;
    if (longsplit) {
      variant = find_variant(XR, 4, 4, 2);
      if (splits <= 0) {
        const long wgs = (long)((M + XR - 1) / XR) * (N / 64);
        splits = (int)(256 / wgs < 1 ? 1 : 256 / wgs);
      }
    } else if (XR == 4 || (tiles < 128 && M <= 16)) {
      // one or two rows on a wide layer: eight waves per tile, two k-blocks in flight
      // each (5% faster than four waves with four at M = 1 on 4096 x 11008 / 12288);
      // narrower layers: eight waves, four k-blocks in flight (timed over graph replays:
      // 2-10% faster than sixteen waves with two on 11008 x 4096 at M = 1-4), two when
      // each wave has fewer than four k-blocks (1024 x 1024, 2560 x 2560: 11-16% faster).
      // Layers with fewer than 128 column tiles take up to 16 rows in blocks of 4 rows,
      // which multiplies the workgroups (3072 x 768 at M = 16: 1.9x faster than one
      // 16-row block split along K)
      variant = wide ? (M <= 2 ? find_variant(4, 1, 8, 2) : find_variant(4, 1, 4, 4))
                     : find_variant(4, 1, 8, K / KBLK >= 32 && XR == 4 ? 4 : 2);
    } else if (XR == 8) {
      // narrow layers with few k-blocks per tile (4096 x 4096): four waves per tile
      // (9% faster than eight over graph replays at M = 8)
      variant = wide ? (ntw == 2 ? find_variant(8, 2, 8, 4) : find_variant(8, ntw, 4, 2))
                     : (longk ? find_variant(8, 1, 8, 4) : find_variant(8, 1, 4, 4));
    } else if (XR == 16) {
      variant = wide ? (ntw == 2 ? find_variant(16, 2, 8, 2) : find_variant(16, ntw, 4, 2))
                     : find_variant(16, 1, 8, 2);
      // 2:4 codes on layers of 128 Mi weights or more: eight column tiles per wave and
      // four waves splitting K (224 workgroups on 8192 x 28672; graph-timed 1.07x over two
      // waves with K in two slices, 1.10x over the 16-row tiled tiles, 1.18x the dense time)
      if (mode == W_SP24 && wide && N % 128 == 0 && (long long)K * N >= (128LL << 20))
        variant = find_variant(16, 8, 4, 2);
      // 2:4 codes on narrow layers: four waves with four k-blocks in flight (each k-block
      // carries 3/4 of the dense bytes; 1.02-1.05x on 4096 x 4096 at M = 16)
      if (mode == W_SP24 && !wide && tiles >= 128) variant = find_variant(16, 1, 4, 4);
    } else if (XR == 32) {
      // narrow layers (one 16-column tile per compute unit or fewer): two blocks of 16 rows,
      // two column tiles per wave, eight waves (graph-timed: 1.11x on 4096 x 4096 and 1.15x
      // on 11008 x 4096 at M = 32 over one 32-row block; the second row block finds the
      // weights in the Infinity Cache).  Wide layers keep one 32-row block.
      variant = wide ? (ntw == 2 ? find_variant(32, 2, 8, 2) : find_variant(32, ntw, 4, 2))
                     : tiles < 128    ? find_variant(16, 1, 8, 2)
                     : (N % 32 == 0 ? find_variant(16, 2, 8, 2) : find_variant(32, 1, 4, 2));
      // 2:4 codes there: four waves with four k-blocks in flight (1.02-1.03x on 4096 x 4096)
      if (mode == W_SP24 && !wide && tiles >= 128 && N % 32 == 0) variant = find_variant(16, 2, 4, 4);
    } else {
      // above 32 rows (layers too small for the tiled kernel): blocks of 16 rows up to 64
      // rows, of 32 above, and the most column tiles per wave (4, 2, 1) that still give
      // at least 128 workgroups.  Measured 1.3-2.6x faster than one 64-row block or the
      // 16-row tiled kernel on 1024 x 1024, 2560 x 2560, 3072 x 768 and 4096 x 4096 (2:4)
      // at M = 48-128
      const int xr = M <= 64 ? 16 : 32;
      const long mb = (M + xr - 1) / xr;
      int nt = 1;
      for (int c : {4, 2}) {
        if (N % (16 * c) == 0 && mb * (tiles / c) >= 128) {
          nt = c;
          break;
        }
      }
      variant = nt == 4 ? find_variant(xr, 4, 4, 2)
                        : (xr == 16 ? find_variant(16, nt, 8, 2) : find_variant(32, nt, 4, 2));
    }
    if (fp8_one) {
      if (XR == 8 && wide) variant = find_variant(8, 1, 4, 4);
      if (XR == 16 && wide) variant = find_variant(16, 1, 8, 2);
      if (XR == 32) variant = wide ? find_variant(32, 1, 4, 2) : find_variant(32, 1, 8, 2);
    }
  }
  if (variant < 0 || variant >= kNumVariants) return -8;
  const Variant& v = kVariants[variant];
  if (N % (16 * v.NT) != 0) return -2;
  const int Gk = K / KBLK;
  const int MT = (v.XR + 15) / 16;
  // buffer descriptors and the offsets through them are 32-bit: the X rows of one block,
  // and the weight bytes of one workgroup's column tiles, must stay below 2 GiB
  const long long lim = 1LL << 31;
  if ((long long)v.XR * K * x_elem_bytes(mode) >= lim) return -2;
  const long long wbytes = mode == W_FP16 ? (long long)v.NT * 16 * K * 2
                           : mode == W_SP24 ? (long long)v.NT * Gk * 512
                                            : (long long)v.NT * Gk * 1024;
  if (wbytes >= lim) return -2;
  p->variant = variant;
  p->mode = mode;
  p->MT = MT;
  p->NT = v.NT;
  p->WK = v.WK;
  p->mblocks = (M + v.XR - 1) / v.XR;
  p->nblocks = N / (16 * v.NT);
  int maxs = Gk / v.WK;
  if (maxs < 1) maxs = 1;
  if (splits <= 0) {
    // split K only when the workgroups would leave most of the chip idle: the hand-off
    // of the partial sums costs more than partly idle compute units (measured: 192
    // four-tile workgroups beat 384 split ones by 2x on 4096 x 12288; 48 workgroups on
    // 3072 x 768 beat 144 split ones by 2.1x; no split won on any other decode or small
    // layer than the long-K ones above)
    const long base = (long)p->mblocks * p->nblocks;
    const long target = 256;
    long sp = base >= 32 ? 1 : (target + base - 1) / base;
    splits = (int)(sp < 1 ? 1 : sp);
  }
  if (splits > maxs) splits = maxs;
  if (splits < 1) splits = 1;
  if ((long long)Gk * splits >= (1LL << 31)) return -2;  // the kernel's slice bounds are 32-bit
  p->splits = splits;
  if ((long long)p->mblocks * p->nblocks * splits >= lim) return -2;
  p->wgs = p->mblocks * p->nblocks * splits;
  p->threads = 64 * v.WK;
  p->part_floats = splits > 1 ? (size_t)p->mblocks * p->nblocks * splits * v.NT * MT * 256 : 0;
  p->counters = splits > 1 ? p->mblocks * p->nblocks : 0;
  return 0;
}

hipError_t skinny_launch(const SkinnyPlan& p, const uint16_t* X, const void* w,
                         const uint16_t* sp, const uint32_t* zp, uint16_t* Y, float* part,
                         int* counters, int M, int N, int K, int group, hipStream_t st,
                         const float* xscale) {
  (void)group;  // the repacked layout stores one scale row per 128-row block
  const Variant& v = kVariants[p.variant];
  KernelFn fn = p.mode == W_FP16     ? v.f16
               : p.mode == W_ASYM   ? v.asym
               : p.mode == W_SP24   ? v.sp24
               : p.mode == W_SYM64  ? v.sym64
               : p.mode == W_ASYM64 ? v.asym64
               : p.mode == W_SYMB   ? v.symb
               : p.mode == W_ASYMB  ? v.asymb
               : p.mode == W_SYM8   ? v.sym8
               : p.mode == W_ASYM8  ? v.asym8
               : p.mode == W_SYMB64 ? v.symb64
               : p.mode == W_ASYMB64 ? v.asymb64
               : p.mode == W_SYM8G64 ? v.sym8g64
               : p.mode == W_ASYM8G64 ? v.asym8g64
                                    : v.sym;
  hipLaunchKernelGGL(fn, dim3(p.wgs), dim3(p.threads), 0, st, X,
                     reinterpret_cast<const uint4*>(w), sp, reinterpret_cast<const uint2*>(zp), Y,
                     part, counters, M, N, K, p.splits, p.nblocks, xscale);
  return hipGetLastError();
}

}  // namespace w4a16
