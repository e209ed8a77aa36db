// Internal declarations shared by the HIP translation units of libw4a16.
//
// Repacked weight layout (layout version 1), own design for gfx950:
//   A "block" covers 16 output columns (a tile t: n = 16t .. 16t+15) and 128
//   consecutive K (a k-block kb: k = 128kb .. 128kb+127) and takes 1 KiB.
//   Blocks are stored tile-major, K fastest: block index = t * (K/128) + kb.
//   Inside a block, lane l (0..63) of a wave owns bytes [16l, 16l+16): four
//   32-bit words, word j (0..3) holding the 8 codes of column 16t + (l % 16)
//   for rows k = 128kb + 32j + 8(l/16) + e, e = 0..7.  A word therefore holds
//   exactly the 8 K-values one lane feeds to one v_mfma_f32_16x16x32_f16 as its
//   B operand, and one 16-byte load per lane fetches the operands of the four
//   MFMAs that cover the 128-row block.
//   Inside a word, row e sits at nibble pos(e) = e/2 + 4*(e%2), i.e. nibbles
//   hold rows [0,2,4,6,1,3,5,7]; then (word & 0x000F000F) holds the pair
//   (row 0, row 1) in its two 16-bit halves, (word & 0x00F000F0) the pair
//   (2, 3) scaled by 16, and the same two masks on word >> 8 give (4, 5) and
//   (6, 7).  Each such half becomes an exact fp16 by OR-ing in 0x6400 (1024.0),
//   see dequant_word() in gemm_skinny.hip.
//   Because 8 consecutive K of one column always sit in one canonical word
//   (canonical words pack rows 8i..8i+7), every repacked word is one canonical
//   word with its nibbles permuted.
//
// Scales, SH rows per 128-row block (SH = 2 for a group of 64 rows, else 1) so that the
// kernels never divide by the group:
//   sp[((t * Gk + kb) * 16 + c) * SH + h] = s[(128 kb + 64 h) / group][16t + c],
//   Gk = K/128 (fp16 bits); a group of 256 or more rows is stored once per 128-row
//   block it spans; with groups of 64 the two halves of a column sit side by side.
// Zero-points, likewise: zp32[((t * Gk + kb) * SH + h) * 2 + w] =
//   z[(128 kb + 64 h) / group][2t + w], i.e. the 16 zero-points of a tile as one 64-bit
//   word per half, nibble c = column 16t+c.  Half h covers rows 64h .. 64h + 63 of the
//   block: the words j = 2h, 2h + 1 of a lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

constexpr int KBLK = 128;   // K rows per repacked block
constexpr int NTILE = 16;   // columns per repacked tile
constexpr int LAYOUT_VERSION = 1;

// Position of row e (0..7 within a canonical word) inside a repacked word.
__host__ __device__ constexpr int nib_pos(int e) { return (e >> 1) + 4 * (e & 1); }

// ---- launchers (each validates nothing; the C ABI layer validated already) ----
hipError_t launch_repack(const int32_t* q, const uint16_t* s, const int32_t* z,
                         uint32_t* wp, uint16_t* sp, uint32_t* zp,
                         int K, int N, int group, hipStream_t st);
hipError_t launch_unpack(const uint32_t* wp, const uint16_t* sp, const uint32_t* zp,
                         int32_t* q, uint16_t* s, int32_t* z,
                         int K, int N, int group, hipStream_t st);
// 2:4 sparse compress (counts runs with more than two non-zero codes into *bad)
// and its inverse; scales are repacked as for the dense layout.
hipError_t launch_sparse_compress(const int32_t* q, const uint16_t* s, uint32_t* vp,
                                  uint32_t* meta, uint16_t* sp, int* bad, int K, int N, int group,
                                  hipStream_t st);
hipError_t launch_sparse_decompress(const uint32_t* vp, const uint32_t* meta, const uint16_t* sp,
                                    int32_t* q, uint16_t* s, int K, int N, int group,
                                    hipStream_t st);
// MXFP4: canonical E2M1 codes (int32 [K/8, N], 8 along K) and E8M0 scales (bytes
// [K/32, N]) -> 1 KiB code blocks [N/16][K/128] (lane l: column l%16, rows 32(l/16) ..
// +31, two codes per byte, low nibble first) and scale blocks [N/16][K/128][64 bytes]
// (byte l: the scale of lane l's 32 rows).
hipError_t launch_mx_repack(const int32_t* q, const uint8_t* e, uint32_t* wp, uint8_t* sp,
                            int K, int N, hipStream_t st);
hipError_t launch_dequant(const int32_t* q, const uint16_t* s, const int32_t* z,
                          uint16_t* W, int K, int N, int group, hipStream_t st);
// bf16 X [M][K] -> fp16 Xh [M][K] = X * 2^d per row, rscale[row] = 2^-d (bf16_rows.hip)
hipError_t launch_bf16_rows_to_f16(const uint16_t* X, uint16_t* Xh, float* rscale, int M, int K,
                                   hipStream_t st);
// fp8 E4M3 codes [elems] -> fp16 Xh [elems], exact (bf16_rows.hip); elems % 16 == 0
hipError_t launch_fp8_rows_to_f16(const uint8_t* X8, uint16_t* Xh, size_t elems, hipStream_t st);

// Fused skinny GEMM.  `part` / `counters` form the split-K workspace.
// weight format of a launch; the *64 modes are the same formats with groups of 64 rows,
// the *B modes take bf16 activations and write bf16 outputs, the *8 modes take fp8
// (OCP E4M3) activations with an optional fp32 scale per row and write fp16 outputs;
// W_*B64 and W_*8G64 are those two with groups of 64 rows (skinny kernel only)
enum WMode {
  W_SYM = 0, W_ASYM = 1, W_FP16 = 2, W_SP24 = 3, W_SYM64 = 4, W_ASYM64 = 5, W_SYMB = 6,
  W_ASYMB = 7, W_SYM8 = 8, W_ASYM8 = 9, W_SYMB64 = 10, W_ASYMB64 = 11, W_SYM8G64 = 12,
  W_ASYM8G64 = 13,
  // MXFP4 weights (E2M1 codes, one E8M0 scale per 32 rows along K) with fp8 activations;
  // the scales go to the block-scaled matrix instruction (tiled kernel only)
  W_MX4 = 14
};
__host__ __device__ constexpr bool mode_asym(int m) {
  return m == W_ASYM || m == W_ASYM64 || m == W_ASYMB || m == W_ASYM8 || m == W_ASYMB64 ||
         m == W_ASYM8G64;
}
__host__ __device__ constexpr bool mode_g64(int m) {
  return m == W_SYM64 || m == W_ASYM64 || m == W_SYMB64 || m == W_ASYMB64 || m == W_SYM8G64 ||
         m == W_ASYM8G64;
}
__host__ __device__ constexpr bool mode_bf16(int m) {
  return m == W_SYMB || m == W_ASYMB || m == W_SYMB64 || m == W_ASYMB64;
}
__host__ __device__ constexpr bool mode_fp8(int m) {
  return m == W_SYM8 || m == W_ASYM8 || m == W_SYM8G64 || m == W_ASYM8G64 || m == W_MX4;
}
// 64 scale bytes per 1 KiB code block: two fp16 rows (groups of 64) or the 64 E8M0 bytes
// of MXFP4 (one per lane of the block)
__host__ __device__ constexpr bool mode_scale64(int m) { return mode_g64(m) || m == W_MX4; }
// packed 4-bit codes with scales (and zero-points): the dense repacked formats
__host__ __device__ constexpr bool mode_dense4(int m) {
  return m != W_FP16 && m != W_SP24 && m >= 0 && m <= W_MX4;
}
struct SkinnyPlan {
  int variant;   // index into the variant table
  int mode;      // WMode
  int MT, NT, WK;
  int splits;
  int mblocks, nblocks;
  int wgs, threads;
  size_t part_floats;  // workspace floats needed for partials
  int counters;        // workspace ints needed for arrival counters
};
int skinny_variant_count();
const char* skinny_variant_name(int v);
// Fills `p` for a shape; variant < 0 or splits <= 0 mean automatic.  Returns 0 or a
// negative W4A16 error code for an unusable (variant, shape) pair.
int skinny_make_plan(int M, int N, int K, int group, int mode, int variant, int splits,
                     SkinnyPlan* p);
// w: repacked codes (W_SYM / W_ASYM) or fp16 Wt[N][K] (W_FP16, sp = zp = NULL).
// X holds fp8 codes (one byte per element) in the fp8 modes; xscale is their optional
// per-row fp32 scale (NULL: 1), ignored by every other mode.
hipError_t skinny_launch(const SkinnyPlan& p, const uint16_t* X, const void* w,
                         const uint16_t* sp, const uint32_t* zp, uint16_t* Y, float* part,
                         int* counters, int M, int N, int K, int group, hipStream_t st,
                         const float* xscale = nullptr);

// Tiled GEMM for larger M (packed weights, dense or 2:4, and the fp16 baseline).  Tile geometry and the
// data-parallel / stream-K work split are fixed by the plan.
struct TiledArgs {
  int M, N, K;
  int tiles_m, tiles_n, group_m;
  int grid;        // persistent workgroups
  int dp_rounds;   // rounds of whole tiles handed out data-parallel
  long long sk_units;   // (tile, k-block) units of the remaining tiles
  long long sk_per_wg;  // units per workgroup stripe
  const float* xscale;  // fp32 scale per row of X (nullptr: 1): fp8 activations, or rows
                        // rewritten in fp16 (the inverse power of two of bf16 rows, the
                        // caller's scale of fp8 rows)
  int out_bf16;         // bf16 activations: Y is written in bf16 (else fp16)
};
struct TiledPlan {
  int variant;  // index into the tiled variant table
  int mode;     // WMode
  TiledArgs args;
  int wgs, threads;
  size_t part_floats;  // workspace floats for partial tiles (two slots per workgroup)
  int fixup_wgs;       // workgroups of the second pass (stream-K tiles x row tiles), 0 if none
};
// The fp16 baseline (W_FP16) has its own variant table; the packed formats share one.
// MXFP4 x fp8 for M <= 32: weights streamed straight to registers, 4 waves split K
int mx_decode_variant_count();
const char* mx_decode_variant_name(int v);
hipError_t mx_decode_launch(int variant, const uint8_t* X, const float* xscale, const void* wp,
                            const uint8_t* sp, uint16_t* Y, int M, int N, int K, hipStream_t st);
int tiled_variant_count(int mode);
const char* tiled_variant_name(int mode, int v);
// variant < 0: automatic; grid <= 0: automatic number of workgroups.
int tiled_make_plan(int M, int N, int K, int mode, int variant, int grid, TiledPlan* p);
// X holds fp8 codes in the fp8 modes, with xscale their optional per-row scale.
// rows16 (dense fp16 modes): X holds bf16 or fp8 rows rewritten in fp16
// (launch_bf16_rows_to_f16 / launch_fp8_rows_to_f16) and xscale, if not NULL, scales each
// row's finished sums; bf16_out: Y is written in bf16.
hipError_t tiled_launch(const TiledPlan& p, const uint16_t* X, const void* w, const uint16_t* sp,
                        const uint32_t* zp, uint16_t* Y, float* part, hipStream_t st,
                        const float* xscale = nullptr, bool rows16 = false,
                        bool bf16_out = false);

// Calibration kernels (probes.hip).
hipError_t launch_probe_read(const void* p, size_t bytes, uint32_t* out, hipStream_t st);
hipError_t launch_probe_mfma(int workgroups, int iters, float* out, hipStream_t st);
double probe_mfma_flops(int workgroups, int iters);

}  // namespace w4a16
