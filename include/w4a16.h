/*
 * w4a16.h -- C ABI of the MI355X (gfx950) W4A16 mixed-precision GEMM library.
 *
 * Computes Y[M,N] = X[M,K] * dequant(W), X and Y fp16, W 4-bit codes with one
 * fp16 scale (and optionally one 4-bit zero-point) per group of `group`
 * consecutive K per output column, accumulated in fp32.
 *
 * Pages this interface follows (all three describe the Marlin FP16xINT4 kernel):
 *   [P1] "Marlin", Spark Notes, dingiv.github.io/ai/compute/kernel/marlin
 *   [P2] "Marlin / GPTQ-Marlin", brain.gartu.xyz/ia/llm/quantification/optimisations/marlin/
 *   [P3] "Marlin Project Overview", vecbase.com/en/p/IST-DASLab/marlin
 *
 * General rules for every entry point below:
 *   - Pointers named as "device" must be device memory on the current HIP
 *     device (hipMalloc, or a torch CUDA tensor).  The caller allocates and
 *     frees every buffer it passes; the library never frees caller memory.
 *   - fp16 values travel as uint16_t bit patterns.  All arrays are dense
 *     row-major with no padding.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued
 *     asynchronously on it; no entry point synchronizes the host, except
 *     w4a16_sparse24_repack (see there).
 *   - Arguments are validated synchronously on the host before anything is
 *     enqueued; on error nothing is enqueued and a negative code is returned.
 *     Faults inside a kernel surface at the caller's next synchronization.
 *   - Functions are thread-safe.  Concurrent calls on different streams are
 *     safe; the library keeps one reduction workspace per (device, stream).
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------------- */
#define W4A16_OK              0
#define W4A16_ERR_NULL       -1  /* a required pointer is NULL                      */
#define W4A16_ERR_SHAPE      -2  /* M,N,K <= 0; K % 128; K % group; group not 64 or 128j; N % 16 ... */
#define W4A16_ERR_ALIGN      -3  /* a pointer is not 16-byte aligned                */
#define W4A16_ERR_DEVICE     -4  /* no HIP device, or the current device is not gfx950 */
#define W4A16_ERR_LAUNCH     -5  /* the HIP runtime reported a launch error         */
#define W4A16_ERR_WORKSPACE  -6  /* the reduction workspace could not be allocated  */
#define W4A16_ERR_NOT24      -7  /* sparse repack input is not 2:4 along K          */
#define W4A16_ERR_ARG        -8  /* an enumerated argument is out of range          */

/* Layout version of the repacked buffers produced by w4a16_repack and
 * w4a16_sparse24_repack.  Stored blobs from a different version must be
 * repacked again from the canonical format. */
int w4a16_layout_version(void);

/* Static English description of a return code (never NULL). */
const char* w4a16_strerror(int code);

/* ---- sizes ------------------------------------------------------------------- */
#define W4A16_BUF_W        0  /* dense repacked codes         : K*N/2 bytes              */
#define W4A16_BUF_S        1  /* dense repacked scales        : 2*(K/128)*N bytes (x2 for group 64) */
#define W4A16_BUF_Z        2  /* dense repacked zero-points   : (K/128)*N/2 bytes (x2 for group 64) */
#define W4A16_BUF_SPARSE_V 3  /* 2:4 kept codes               : K*N/4 bytes              */
#define W4A16_BUF_SPARSE_I 4  /* 2:4 position metadata        : K*N/8 bytes              */
#define W4A16_BUF_SPARSE_S 5  /* 2:4 repacked scales          : 2*(K/128)*N bytes        */
/* (repacked scales and zero-points hold one row per 128 rows of K, so a group of
 *  256 or more rows is stored once per 128-row block it spans; with groups of 64
 *  rows they hold two rows per block.  The 2:4 buffers need group % 128 == 0 and are
 *  0 bytes for group 64.) */
/* Bytes of buffer `which` for a K x N weight; 0 if the shape is invalid. */
size_t w4a16_packed_bytes(int K, int N, int group, int which);

/* ---- offline repack ([P2] "2. Tiled layout et repacking"; [P3] "Key Techniques",
 *      reshuffling of weights and scales) -------------------------------------------
 * Converts the canonical group-quantized format into the kernel layout, once,
 * at load time; inference never touches the canonical format again.
 *
 *   q  (device, in)  int32 [K/8][N]: 8 codes per word packed along K,
 *                    nibble j of q[i][n] is the code of row 8i+j (unsigned).
 *   s  (device, in)  fp16  [K/group][N]: scale of (group, column).
 *   z  (device, in)  int32 [K/group][N/8] packed along N (nibble j of z[G][c]
 *                    is the zero-point of column 8c+j), or NULL for the
 *                    symmetric format (zero-point 8).
 *   wp (device, out) W4A16_BUF_W bytes; sp (device, out) W4A16_BUF_S bytes;
 *   zp (device, out) W4A16_BUF_Z bytes, must be NULL exactly when z is NULL.
 * Shape rules: K > 0, N > 0, K % 128 == 0, group == 64 or group % 128 == 0,
 * K % group == 0, N % 16 == 0.  All pointers 16-byte aligned.  Input and output must
 * not overlap.
 */
int w4a16_repack(const int32_t* q, const uint16_t* s, const int32_t* z,
                 void* wp, uint16_t* sp, void* zp,
                 int K, int N, int group, void* stream);

/* Exact inverse of w4a16_repack (for round-trip checks): rewrites q, s and,
 * when zp is not NULL, z in the canonical format.  Same shapes and rules. */
int w4a16_unpack(const void* wp, const uint16_t* sp, const void* zp,
                 int32_t* q, uint16_t* s, int32_t* z,
                 int K, int N, int group, void* stream);

/* ---- fused GEMM ([P1] "反量化与 GEMM 融合", "Striped 划分与流水线";
 *      [P2] "Architecture générale"; [P3] "Key Techniques") --------------------------
 * Y = X * W with W = (q - z) * s never written to memory: packed codes are read
 * from HBM once, turned into fp16 in registers, multiplied on the matrix cores
 * with fp32 accumulation, and Y is rounded once to fp16 (nearest-even).
 *
 *   X  (device, in)  fp16 [M][K];  wp, sp, zp as produced by w4a16_repack
 *                    (zp NULL for the symmetric format);
 *   Y  (device, out) fp16 [M][N], fully overwritten.
 * Shape rules: M >= 1 plus the repack rules.  X, Y, wp, sp, zp 16-byte aligned.
 * Results are bitwise reproducible from run to run for a given shape.
 * The first call for a (device, stream) may allocate the reduction workspace
 * (hipMalloc, plus a hipMemsetAsync of its counters on `stream`); later calls
 * allocate only when a larger shape needs more, at least doubling it.  A buffer
 * replaced that way is kept until the process ends, never freed, because launches
 * in flight and HIP graphs captured earlier may still use it.  While `stream` is
 * being captured into a graph nothing is allocated: a call whose plan needs more
 * workspace than the stream already holds returns W4A16_ERR_WORKSPACE and enqueues
 * nothing.  So make one call of each shape (or a larger one) on the stream before
 * capturing it, or hand the stream a buffer with w4a16_set_workspace.  A captured
 * graph keeps using the workspace it was captured with, and graphs replayed
 * concurrently on one stream's workspace race.
 */
int w4a16_gemm(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
               uint16_t* Y, int M, int N, int K, int group, void* stream);

/* ---- the same GEMM without any allocation, for callers that cannot allocate: code
 *      under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc ----
 * w4a16_gemm_noalloc: w4a16_gemm with the same arguments, rules, automatic plans, kernels
 *   and results (bit for bit), except where the split-K / stream-K workspace lives: a
 *   fixed scratch array of W4A16_NOALLOC_SCRATCH_BYTES in the library's device memory
 *   (one per device, held until the process ends; the first W4A16_WS_COUNTER_BYTES are
 *   arrival counters, the rest fp32 partials) instead of a per-stream buffer.  The call
 *   never allocates or frees memory and issues no memset.  Its first call on a device
 *   looks the array up and clears the counters with a small kernel on `stream`; the
 *   kernels leave them at zero again.  Every call on one device shares the array and
 *   finds it as the last call left it: calls that overlap in time on one device (on
 *   different streams, or concurrent replays of graphs holding such calls) race and give
 *   wrong results.  A plan needing more workspace than the array holds returns
 *   W4A16_ERR_WORKSPACE and enqueues nothing (no automatic plan of a valid shape needs
 *   more: the largest takes two 128 x 512 fp32 pieces for each of 256 workgroups). */
#define W4A16_NOALLOC_SCRATCH_BYTES (65536 + (128u << 20))
int w4a16_gemm_noalloc(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                       uint16_t* Y, int M, int N, int K, int group, void* stream);

/* Same as w4a16_gemm with an explicit kernel plan (tuning and tests):
 *   variant : -1 = automatic, else an index < w4a16_gemm_variants();
 *   splits  : 0 = automatic.  For a "skinny_*" variant (one workgroup per
 *             (row block, column block, K slice)), the number of K slices reduced
 *             across workgroups, clamped to the number of 128-row blocks per wave.
 *             For a "tiled_*" variant (persistent workgroups over tiles, the
 *             (tile, k-block) work cut into equal stripes), the number of
 *             workgroups.
 * Automatic plans use the skinny kernel for M <= 32 and the tiled kernel above,
 * except for 33 <= M < 256 on layers with K*N < 32 Mi and N >= 2048 (skinny).
 * The same variants and rules apply to the 2:4 format (w4a16_sparse24_gemm_plan). */
int w4a16_gemm_plan(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                    uint16_t* Y, int M, int N, int K, int group,
                    int variant, int splits, void* stream);

/* Number of fused-kernel variants, and a static name for one (NULL if out of range). */
int w4a16_gemm_variants(void);
const char* w4a16_gemm_variant_name(int variant);

/* Bytes of device workspace the automatic plans of w4a16_gemm, w4a16_sparse24_gemm,
 * w4a16_fp16_gemm, w4a16_gemm_bf16, w4a8_gemm and w4a8_mx_gemm need for an (M, N, K) GEMM
 * on one stream (the largest over the entry points; 0 when no plan for the shape reduces
 * across workgroups or rewrites its activations, or for an invalid shape).  Above 32 rows
 * this includes w4a16_gemm_bf16's fp16 copy of X (M*K*2 bytes) and its M fp32 row scales.  The library allocates this itself, per (device, stream), on the first call
 * that needs it and keeps it for later calls; the query lets a caller budget device
 * memory ahead of time.  Host only. */
size_t w4a16_workspace_bytes(int M, int N, int K);

/* Caller-owned workspace (the pages leave workspace ownership open; this lets a caller such
 * as a framework allocator own all device memory).  Hands the library the device buffer
 * ptr of `bytes` bytes to use, instead of allocating its own, for every GEMM launched on
 * `stream` on the current device.  Layout: the first W4A16_WS_COUNTER_BYTES hold the
 * split-K arrival counters, the rest the fp32 partial sums; bytes >= that prefix plus
 * w4a16_workspace_bytes(M, N, K) covers every automatic plan of a shape.  The call
 * clears the counter prefix (hipMemsetAsync on `stream`, so it must not be captured into a
 * graph); the kernels leave the counters at zero again, so no later call clears anything.
 * The library never frees ptr; the caller keeps it alive, and does not use it otherwise,
 * until it is replaced or until ptr = NULL hands the stream back to library-owned
 * workspaces.  Replacing a caller-owned buffer first waits for the stream to drain, so the
 * caller may free the old one once this returns (graphs captured with it must then not be
 * replayed); a buffer the library had allocated for the stream is kept, not freed.  A
 * launch on the stream whose plan needs more than the buffer holds returns
 * W4A16_ERR_WORKSPACE.  Errors: W4A16_ERR_ALIGN (ptr not 256-byte aligned),
 * W4A16_ERR_WORKSPACE (ptr non-NULL with bytes below W4A16_WS_COUNTER_BYTES + 256, or
 * `stream` being captured into a graph), W4A16_ERR_DEVICE, W4A16_ERR_LAUNCH (the clearing
 * or the wait failed). */
#define W4A16_WS_COUNTER_BYTES 65536
int w4a16_set_workspace(void* ptr, size_t bytes, void* stream);

/* Describe the automatic plan for a shape: out[0] = variant, out[1] = the splits
 * value that reproduces it in w4a16_gemm_plan,
 * out[2] = workgroups launched, out[3] = threads per workgroup.  Host only. */
int w4a16_gemm_describe(int M, int N, int K, int group, int* out4);

/* ---- unfused baseline ([P1] "反量化与 GEMM 融合": dequantize, write back, then
 *      a plain GEMM; [P2] "Le problème") ---------------------------------------------
 * w4a16_dequant: Wt (device, out) fp16 [N][K] with Wt[n][k] = RNE((q[k][n] -
 *   z[k/group][n]) * s[k/group][n]) from the canonical q, s, z (z NULL =
 *   symmetric).  Wt is stored output-major like a torch Linear weight.  Shape
 *   rules as w4a16_repack.
 * w4a16_fp16_gemm: Y (device, out) fp16 [M][N] = X [M][K] * Wt[N][K]^T with
 *   fp32 accumulation.  Rules: M, N, K >= 1, K % 128 == 0, N % 16 == 0, 16-byte
 *   aligned pointers.  Uses the same per-stream workspace as w4a16_gemm and the
 *   same kernel choice (skinny kernel for small batches, tiled kernel with fp16
 *   weight tiles for the larger ones, by the rule of w4a16_gemm_plan). */
int w4a16_dequant(const int32_t* q, const uint16_t* s, const int32_t* z, uint16_t* Wt,
                  int K, int N, int group, void* stream);
int w4a16_fp16_gemm(const uint16_t* X, const uint16_t* Wt, uint16_t* Y,
                    int M, int N, int K, void* stream);
/* w4a16_fp16_gemm with an explicit plan: variant -1 = automatic, else an index <
 * w4a16_fp16_gemm_variants(); the skinny variants come first (same names as for
 * w4a16_gemm), then the fp16 tiled ones ("tiled_f16_*"); `splits` as in
 * w4a16_gemm_plan.  Names are static strings (NULL if out of range). */
int w4a16_fp16_gemm_plan(const uint16_t* X, const uint16_t* Wt, uint16_t* Y,
                         int M, int N, int K, int variant, int splits, void* stream);
int w4a16_fp16_gemm_variants(void);
const char* w4a16_fp16_gemm_variant_name(int variant);

/* ---- 2:4 structured sparsity ([P1] "支持 2:4 稀疏加速"; [P2] "4. Support de la
 *      sparsité 2:4") ----------------------------------------------------------------
 * Weights whose every aligned run of 4 rows (along K) per column holds at most two
 * non-zero codes (zero = code 8, symmetric format only) are stored as the two kept
 * codes per run plus their 2-bit positions, and multiplied on the gfx950 sparse
 * matrix instructions (v_smfmac_f32_16x16x64_f16): half the code bytes, half the
 * matrix work.
 *
 * w4a16_sparse24_repack: compress the canonical q (same format as w4a16_repack, z
 *   implied 8) into vp (W4A16_BUF_SPARSE_V bytes, kept codes), idx
 *   (W4A16_BUF_SPARSE_I bytes, positions) and sp (W4A16_BUF_SPARSE_S bytes, scales).
 *   Kept positions are the non-zero ones, topped up with the lowest free positions.
 *   This call synchronizes `stream`: it returns W4A16_ERR_NOT24 when some run holds
 *   more than two non-zero codes (the outputs are then incomplete).  Offline step.
 * w4a16_sparse24_unpack: exact inverse: rewrites the canonical q (code 8 at pruned
 *   positions) and s.
 * w4a16_sparse24_gemm: Y = X * W from the compressed weights, same rules and
 *   guarantees as w4a16_gemm (idx 16-byte aligned as well).
 * w4a16_sparse24_gemm_plan: the same with an explicit plan, as w4a16_gemm_plan.
 * The 2:4 format takes groups that are whole multiples of 128 rows (W4A16_ERR_SHAPE
 * for group 64).
 * Shape rules as w4a16_repack. */
int w4a16_sparse24_repack(const int32_t* q, const uint16_t* s, void* vp, void* idx,
                          uint16_t* sp, int K, int N, int group, void* stream);
int w4a16_sparse24_unpack(const void* vp, const void* idx, const uint16_t* sp,
                          int32_t* q, uint16_t* s, int K, int N, int group, void* stream);
int w4a16_sparse24_gemm(const uint16_t* X, const void* vp, const void* idx,
                        const uint16_t* sp, uint16_t* Y, int M, int N, int K, int group,
                        void* stream);
int w4a16_sparse24_gemm_plan(const uint16_t* X, const void* vp, const void* idx,
                             const uint16_t* sp, uint16_t* Y, int M, int N, int K, int group,
                             int variant, int splits, void* stream);

/* ---- bf16 activations ---------------------------------------------------------------
 * w4a16_gemm_bf16: Y (device, out) bf16 [M][N] = X (device, in) bf16 [M][K] * dequant(W),
 *   same repacked weights and rules as w4a16_gemm (groups of 64 rows included), Y rounded
 *   once to bf16 (nearest-even).  Bitwise reproducible like w4a16_gemm.  Two paths:
 *   - skinny kernel (up to 32 rows, and where w4a16_gemm keeps the skinny kernel): the
 *     weights enter the bf16 matrix instructions as the exact integers 128 + q; the offset
 *     128 + z is removed with the block's activation row sums and the scale applied in
 *     fp32 per 128-row block (per 64-row half for groups of 64).  Those fp32 sums carry
 *     every activation times 128 + q, so one activation far above the rest of its row
 *     (beyond about 2^18 times) costs accuracy in outputs whose weight at its position is
 *     small;
 *   - above: each row of X is first rewritten in fp16 as X * 2^d, with the power of two d
 *     chosen from the row's largest finite magnitude (exact for every value within 2^32 of
 *     it; smaller ones round to the fp16 subnormal grid), then the fp16 tiled kernel of
 *     w4a16_gemm runs and applies 2^-d to each finished fp32 sum before the bf16 store.
 *     The fp16 rows live in the per-stream workspace (M*K*2 bytes more, counted by
 *     w4a16_workspace_bytes).
 * w4a16_gemm_bf16_plan: the same with an explicit variant < w4a16_gemm_bf16_variants():
 *   the skinny variants, then the bf16 tiled variants (indices as in w4a16_gemm_plan; the
 *   eight-wave ones, and any of them with groups of 64 rows, return W4A16_ERR_ARG; the
 *   weights enter as 128 + q and the offset and scale are applied per k-block in fp32,
 *   as in the skinny path), then the fp16 tiled variants on rewritten rows ("rows16_*");
 *   `splits` as in w4a16_gemm_plan (for a tiled variant: workgroups).
 * w4a16_gemm_bf16_variants / _variant_name: their number, and a static name for one
 *   (NULL if out of range). */
int w4a16_gemm_bf16(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                    uint16_t* Y, int M, int N, int K, int group, void* stream);
int w4a16_gemm_bf16_plan(const uint16_t* X, const void* wp, const uint16_t* sp, const void* zp,
                         uint16_t* Y, int M, int N, int K, int group, int variant, int splits,
                         void* stream);
int w4a16_gemm_bf16_variants(void);
const char* w4a16_gemm_bf16_variant_name(int variant);

/* ---- fp8 activations: W4A8 ---------------------------------------------------------
 * INT4 weights times FP8 activations, the mixed-precision variant that runs the product
 * on FP8 matrix units (dingiv.github.io "Marlin", section "CUTLASS W4A8（混合精度）").
 * w4a8_gemm: Y (device, out) fp16 [M][N] = diag(a) * X (device, in) * dequant(W), with
 *   X8     (device, in)  [M][K] bytes, OCP FP8 E4M3 codes (bias 7, no infinities;
 *          S.1111.111 is NaN, and NaN inputs give unspecified outputs), row-major;
 *   xscale (device, in)  fp32 [M], the scale a[m] of activation row m, or NULL for 1;
 *          4-byte aligned (W4A16_ERR_ALIGN otherwise);
 *   wp, sp, zp           the repacked weights of w4a16_repack (zp NULL: symmetric, z = 8);
 *   group  as for w4a16_gemm: 64, or a multiple of 128 dividing K.
 *   Every other rule (shapes, 16-byte alignment of X8, wp, sp, zp and Y, error codes,
 *   asynchronous execution on `stream`, library-owned workspace, Y fully overwritten) is
 *   that of w4a16_gemm.  Bitwise reproducible like w4a16_gemm.  Two paths:
 *   - skinny kernel (up to 32 rows, and where w4a16_gemm keeps the skinny kernel): the
 *     weights enter v_mfma_f32_16x16x32_fp8_fp8 as the exact E4M3 integers q - z, the
 *     scale s applies in fp32 per 128-row block (per 64-row half for groups of 64), and
 *     a[m] in fp32 before the one rounding of Y to fp16 (nearest-even);
 *   - above: the codes are first rewritten as fp16 (every E4M3 value is one, so this is
 *     exact; M*K*2 bytes of workspace, counted by w4a16_workspace_bytes), then the fp16
 *     tiled kernel of w4a16_gemm runs (weights RNE_fp16((q - z) * s), fp32 sums) and
 *     applies a[m] to each finished sum before the rounding of Y.  On gfx950 this is
 *     faster than the fp8 matrix instructions there, whose per-block fp32 rescale and
 *     E4M3 conversion of every weight keep them bound by the vector unit.
 * w4a8_gemm_plan: the same with an explicit variant and `splits`, numbered like
 *   w4a16_gemm_bf16_plan (w4a16_gemm_bf16_variants / _variant_name give the count and
 *   names): the skinny variants; the fp8 tiled variants (v_mfma_scale_f32_16x16x128_f8f6f4
 *   with unit block scales, the weights as E4M3 integers q - z, s per block in fp32; they
 *   need an even number of 16-row tiles, so not "tiled_bm16_*", and groups of 128 rows or
 *   more, else W4A16_ERR_ARG); then the fp16 tiled variants on rewritten rows
 *   ("rows16_*", every group). */
int w4a8_gemm(const uint8_t* X8, const float* xscale, const void* wp, const uint16_t* sp,
              const void* zp, uint16_t* Y, int M, int N, int K, int group, void* stream);
int w4a8_gemm_plan(const uint8_t* X8, const float* xscale, const void* wp, const uint16_t* sp,
                   const void* zp, uint16_t* Y, int M, int N, int K, int group, int variant,
                   int splits, void* stream);

/* ---- MXFP4 weights x fp8 activations: dequantization inside the matrix instruction ---
 * FP4 weights with micro-block scales that the matrix unit applies itself, instead of
 * unpacking the weights in registers first (dingiv.github.io "Marlin", section "与
 * Blackwell NVFP4 的对比").  The format is OCP MXFP4, the micro-block format of gfx950's
 * block-scaled matrix instruction: weight w[k][n] = e2m1(q[k][n]) * 2^(e[k/32][n] - 127),
 * E2M1 codes (sign, 2-bit exponent of bias 1, 1 mantissa bit: +-{0, .5, 1, 1.5, 2, 3, 4,
 * 6}) and one E8M0 scale byte per 32 rows along K (255 is NaN: unspecified outputs).
 * w4a8_mx_repack: one-time layout change, like w4a16_repack:
 *   q  (device, in)  int32 [K/8][N]: code of row k, column n in bits 4(k%8) .. +3 of
 *      word [k/8][n] (the canonical packing of w4a16_repack);
 *   e  (device, in)  uint8 [K/32][N]: E8M0 scale of rows 32b .. 32b+31 of column n;
 *   wp (device, out) K*N/2 bytes: code blocks [N/16][K/128] of 1 KiB, lane l of a block
 *      holding column l%16, rows 32(l/16) .. +31, two codes per byte, low nibble first
 *      (the instruction's operand order; each word is a canonical word, unchanged);
 *   sp (device, out) K*N/32 bytes: scale blocks [N/16][K/128] of 64 bytes, byte l the
 *      scale of lane l's 32 rows.
 *   K % 128 == 0, N % 16 == 0, K*N/8 < 2^31; q, wp, sp 16-byte aligned.  Asynchronous
 *   on `stream`; the caller owns every buffer.
 * w4a8_mx_gemm: Y (device, out) fp16 [M][N] = diag(a) * X (device, in) * W, with X8 and
 *   xscale exactly as in w4a8_gemm and wp, sp from w4a8_mx_repack.  Every kernel runs
 *   v_mfma_scale_f32_16x16x128_f8f6f4 with the codes as the FP4 operand and the lane's
 *   E8M0 byte as its block scale, X as the FP8 operand with unit scale; fp32
 *   accumulation, a[m] in fp32 before the one rounding of Y to fp16 (nearest-even).
 *   M <= 32 runs on the decode kernel (codes streamed straight to registers, one or two
 *   16-row tiles, 4 waves splitting K, summed in LDS in wave order), larger M on the
 *   tiled kernel.
 *   Shapes, 16-byte alignment of X8, wp, sp and Y, error codes, asynchronous execution,
 *   the library-owned (or w4a16_set_workspace) stream-K workspace and bitwise
 *   reproducibility are those of w4a16_gemm.
 * w4a8_mx_gemm_plan: the same with an explicit variant (0 .. w4a8_mx_variants()-1, named
 *   by w4a8_mx_variant_name: first the tiled variants of w4a16_gemm_variants in the same
 *   order, then the decode kernels "mx_decode_nt1/2/4" with 1, 2 or 4 column tiles per
 *   workgroup; -1 = automatic) and, for a tiled variant, `grid` persistent workgroups
 *   (0 = automatic; the decode kernels ignore it).  Tiled variants with an odd number of
 *   16-row tiles, and decode kernels with M > 32, return W4A16_ERR_ARG. */
int w4a8_mx_repack(const int32_t* q, const uint8_t* e, void* wp, void* sp, int K, int N,
                   void* stream);
int w4a8_mx_gemm(const uint8_t* X8, const float* xscale, const void* wp, const void* sp,
                 uint16_t* Y, int M, int N, int K, void* stream);
int w4a8_mx_gemm_plan(const uint8_t* X8, const float* xscale, const void* wp, const void* sp,
                      uint16_t* Y, int M, int N, int K, int variant, int grid, void* stream);
int w4a8_mx_variants(void);
const char* w4a8_mx_variant_name(int variant);

/* ---- calibration kernels (measurement only) ---------------------------------------
 * The achievable ceilings the GEMM's rates are set against, beside the published peaks.
 * w4a16_probe_read: one plain streaming read of `bytes` bytes at device pointer p
 *   (16-byte aligned, bytes a positive multiple of 16) with 16-byte non-temporal loads.
 *   The data is XOR-folded per thread; out (device, one uint32) is written only when a
 *   thread's fold equals 0x9E3779B9, otherwise left untouched.
 * w4a16_probe_mfma: `workgroups` workgroups of 4 waves, each wave running `iters`
 *   rounds of 4 independent v_mfma_f32_32x32x16_f16 on register operands (no memory
 *   traffic); out (device, one float) is never written in practice.
 *   w4a16_probe_mfma_flops gives the flops of such a launch (host only).
 * Both return the usual codes: W4A16_ERR_NULL, W4A16_ERR_SHAPE (read size),
 * W4A16_ERR_ALIGN, W4A16_ERR_ARG (workgroups outside 1..65536 or iters < 1),
 * W4A16_ERR_DEVICE, W4A16_ERR_LAUNCH. */
int w4a16_probe_read(const void* p, size_t bytes, uint32_t* out, void* stream);
int w4a16_probe_mfma(int workgroups, int iters, float* out, void* stream);
double w4a16_probe_mfma_flops(int workgroups, int iters);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_H */
