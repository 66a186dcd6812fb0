/*
 * fp4q -- FP4 microscaling block quantization with block-scale search,
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What the library computes is defined on these web pages (cited by title
 * and section):
 *   [SS]  "Resumo Técnico: ScaleSweep" -- NVFP4 two-level scaling
 *         (Declaração do Problema), the MSE / WMSE objectives (1. Objetivos
 *         de Otimização), the global scale S = max|x| / (256 * 6) and the
 *         bit-pattern window around the AbsMax block scale bounded by
 *         Lemma 4.1 (+7) and Lemma 4.3 (-3, MSE) or the empirical -8 (WMSE)
 *         (2. Limites Teóricos para Varredura Eficiente, 3. Implementação).
 *   [MR]  "Bridging the Gap Between Promise and Performance for Microscaling
 *         FP4 Quantization" -- MXFP4 with power-of-two E8M0 scales
 *         (1. O Problema), MSE-optimised scale grid and fused block Hadamard
 *         micro-rotation (2. Metodologia e Análise, 3. Implementação de
 *         Hardware).
 *   [TQ]  "Resumo Técnico: TORQ" -- MXFP4 activations; the S-step maps the
 *         block maximum onto the largest E2M1 code (B. Rotação de
 *         Alinhamento Micro).
 *   [FC]  "FOCUS: FP4 Optimization via Coupled-Relaxation and
 *         Dual-Granularity Scaling" -- block sizes 16 (NVFP4) and 32
 *         (MXFP4); only the FP4 codes and the dequantization scales are
 *         stored (Declaração do Problema, 4. Implantação e Compatibilidade).
 *
 * Conventions shared by every call
 *   - x is a row-major R x C matrix with leading dimension ld >= C (elements).
 *     Blocks and Hadamard groups run along C.  C must be a multiple of the
 *     block size (and of the Hadamard size).  R * C / 16 must be below 2^31.
 *   - x must be 16-byte aligned and ld * sizeof(element) a multiple of 16.
 *   - Outputs are dense row-major: packed codes have C/2 bytes per row
 *     (element 2k in the low nibble of byte k, element 2k+1 in the high
 *     nibble; a code is (sign << 3) | e2m1_index, index 0..7 for magnitudes
 *     0, 0.5, 1, 1.5, 2, 3, 4, 6); per-block arrays (scales, losses,
 *     offsets) have C/block entries per row.
 *   - Every pointer except the stream is a DEVICE pointer.  The caller owns
 *     every buffer; the library allocates nothing and keeps no state
 *     between calls.
 *   - stream is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; nothing waits on the host.
 *   - Errors in the arguments are returned synchronously, before anything is
 *     enqueued.  Errors in the data (non-finite x, negative or non-finite
 *     importance, an invalid given global scale) are found on the device:
 *     they set bits of the status word, the uint32 at byte 0 of the
 *     workspace (FP4Q_DATA_* below), and leave that call's outputs
 *     unspecified.  After the stream has finished, the word holds exactly
 *     the data errors of the last call on that workspace (0: none); a
 *     fresh, uninitialised workspace is fine.  Bytes 4..7 hold a tag of
 *     the call: the call's first kernel merges its bits into the 64-bit
 *     slot under its dispatch ID (the packet's index in the hardware
 *     queue), replacing a slot left by any earlier call, and later kernels
 *     of the call add bits.  The workspace must be 8-byte aligned.  Calls
 *     that overlap on one workspace (different streams) race on it.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp4q_status {
  FP4Q_OK = 0,
  FP4Q_ERR_NULL = 1,      /* a required pointer is NULL */
  FP4Q_ERR_SHAPE = 2,     /* rows/cols/ld/block/Hadamard size inconsistent */
  FP4Q_ERR_ARG = 3,       /* bad enum, window or flag */
  FP4Q_ERR_ALIGN = 4,     /* x or its row stride not 16-byte aligned */
  FP4Q_ERR_WORKSPACE = 5, /* workspace NULL or smaller than fp4q_workspace_bytes() */
  FP4Q_ERR_HIP = 6        /* a kernel launch failed (hipGetLastError) */
} fp4q_status_t;

/* The *_INT_MIN_ / *_INT_MAX_ enumerators are not values to pass: they make
 * every int a valid value of the enum, so an out-of-range value a caller
 * passes reaches the library's argument checks (FP4Q_ERR_ARG). */
typedef enum fp4q_dtype {
  FP4Q_F32 = 0,
  FP4Q_BF16 = 1,
  FP4Q_DTYPE_INT_MIN_ = -2147483647 - 1,
  FP4Q_DTYPE_INT_MAX_ = 2147483647
} fp4q_dtype_t;
typedef enum fp4q_loss {
  FP4Q_MSE = 0,
  FP4Q_WMSE = 1,
  FP4Q_LOSS_INT_MIN_ = -2147483647 - 1,
  FP4Q_LOSS_INT_MAX_ = 2147483647
} fp4q_loss_t;
typedef enum fp4q_format {
  FP4Q_NVFP4 = 0,
  FP4Q_MXFP4 = 1,
  FP4Q_FORMAT_INT_MIN_ = -2147483647 - 1,
  FP4Q_FORMAT_INT_MAX_ = 2147483647
} fp4q_format_t;

/* flags of fp4q_quantize_nvfp4 */
#define FP4Q_GIVEN_SCALE 0x1u /* read S from *global_scale instead of computing it */
/* Add this call's data errors to the status word instead of replacing it,
 * for chains of calls on one stream that check the word once at the end
 * (the caller zeroes the word before the chain). */
#define FP4Q_ACCUMULATE_STATUS 0x2u

/* bits of the device status word (uint32 at byte 0 of the workspace) */
#define FP4Q_DATA_NONFINITE_INPUT 0x1u  /* x (after rotation) holds Inf or NaN */
#define FP4Q_DATA_BAD_IMPORTANCE 0x2u   /* an importance entry is < 0, Inf or NaN */
#define FP4Q_DATA_BAD_GLOBAL_SCALE 0x4u /* given S is < 0, Inf or NaN */
#define FP4Q_DATA_BAD_SCALE 0x8u        /* fp4q_quantize_relaxed: invalid scale byte or coefficient */
#define FP4Q_DATA_BAD_HESSIAN 0x10u     /* fp4q_gptq_nvfp4: a diagonal entry of U is not finite and > 0 */
#define FP4Q_DATA_BAD_PERM 0x20u        /* fp4q_gptq_static_*: perm is not a permutation of 0 .. cols-1 */

/* Library version as 10000 * major + 100 * minor + patch. */
int fp4q_version(void);

/* Static description of a status code; never NULL. */
const char *fp4q_status_string(fp4q_status_t status);

/* Bytes of device workspace every quantize call needs (a constant).  Bytes
 * 0..3 hold the status word of the last call, 4..7 that call's tag; the
 * rest is scratch the library overwrites. */
size_t fp4q_workspace_bytes(void);

/*
 * NVFP4 quantization with the ScaleSweep block-scale search [SS], optionally
 * after a block Hadamard rotation [MR].
 *
 *   x, dtype, rows, cols, ld  input matrix (FP4Q_F32 or FP4Q_BF16).
 *   importance  [cols] float32 per-column weights (WMSE; NULL for MSE)
 *               ([SS] 1.: importance from input-activation norms or the
 *               Gram diagonal).  With a rotation it must already be in the
 *               rotated basis.
 *   block       16.
 *   loss        FP4Q_MSE or FP4Q_WMSE (WMSE requires importance).
 *   off_lo, off_hi  E4M3 bit-pattern window around the AbsMax base pattern,
 *               -126 <= off_lo <= 0 <= off_hi <= 126 ([SS] 3.: -3, 7 for
 *               MSE; -8, 7 for WMSE; 0, 0 is plain AbsMax round-to-nearest).
 *   hadamard_n  0 (none) or 16, 32, 64, 128: rotate each row's n-column
 *               groups by the orthonormal Sylvester Hadamard matrix first.
 *   flags       0, FP4Q_GIVEN_SCALE and/or FP4Q_ACCUMULATE_STATUS.
 *   codes       [rows * cols / 2] packed E2M1 codes (out).
 *   scales      [rows * cols / 16] E4M3 block-scale bit patterns (out).
 *   global_scale [1] float32 S (out; in with FP4Q_GIVEN_SCALE).
 *   block_loss  [rows * cols / 16] float32 loss of the chosen scale in the
 *               units of x (sum over the block of w * (x - x_hat)^2 in
 *               S-units, times S*S) (out; may be NULL).
 *   offsets     [rows * cols / 16] int8 chosen pattern minus base pattern
 *               (out; may be NULL).
 *   workspace   fp4q_workspace_bytes() bytes of device memory.
 *
 * Computation (every float32 step rounds to nearest even; fused
 * multiply-adds only where written):
 *   S = fp32(max|x| / 1536), S_inv = fp32(1/S) (0 if S = 0);
 *   u = fp32(|x| * S_inv); per block t = fp32(max u / 6);
 *   base = max(1, nearest E4M3 pattern to t, ties to even, saturating 0x7E);
 *   for p = max(1, base+off_lo) .. min(126, base+off_hi): V = E4M3(p),
 *   R = fp32(1/V), q = E2M1 nearest to fp32(u*R) (ties to even index,
 *   saturating at 6), e = fp32(u - q*V); L_p sums the block's terms in
 *   element order with one rounding each: acc = fma(t, e, acc) from 0,
 *   t = e (MSE) or fp32(w*e) (WMSE); the chosen p is the smallest p with
 *   the least L_p.
 */
fp4q_status_t fp4q_quantize_nvfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                  int64_t ld, const float *importance, int block, fp4q_loss_t loss,
                                  int off_lo, int off_hi, int hadamard_n, uint32_t flags,
                                  uint8_t *codes, uint8_t *scales, float *global_scale,
                                  float *block_loss, int8_t *offsets, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * fp4q_quantize_nvfp4 without a workspace, for callers that cannot allocate
 * device memory for one: code being captured into a HIP graph, tight
 * serving loops, harnesses that forbid hipMalloc.  It allocates nothing and
 * calls no allocating routine.
 *
 * Same arguments, computation, errors and results as fp4q_quantize_nvfp4,
 * except that the workspace is replaced by:
 *   status  [2] uint32 device words, 8-byte aligned (out): word 0 receives
 *           the call's data errors (FP4Q_DATA_* bits) and word 1 its tag,
 *           exactly like bytes 0..7 of the workspace (with
 *           FP4Q_ACCUMULATE_STATUS the call adds to word 0).
 * The global-max pass keeps its per-workgroup partials in a static device
 * array of the library instead, fp4q_noalloc_scratch_bytes() = 1 KiB per
 * GPU, held until the process ends.  That is the most the pass ever writes
 * (at most 256 partials whatever the tensor's size), so no input is too
 * large for it.  The array's address on the current device is looked up
 * once per device, on its first call (FP4Q_ERR_HIP if that fails); the
 * current device must be the stream's.  All calls on one GPU share the
 * array: calls that overlap on a GPU (different streams, or threads) race
 * on it and must be serialized by the caller.  Calls in order on one
 * stream are fine: each call writes every partial it reads.
 */
fp4q_status_t fp4q_quantize_nvfp4_noalloc(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                          int64_t ld, const float *importance, int block, fp4q_loss_t loss,
                                          int off_lo, int off_hi, int hadamard_n, uint32_t flags,
                                          uint8_t *codes, uint8_t *scales, float *global_scale,
                                          float *block_loss, int8_t *offsets, uint32_t *status, void *stream);

/* Bytes of the static device scratch of fp4q_quantize_nvfp4_noalloc (per GPU). */
size_t fp4q_noalloc_scratch_bytes(void);

/*
 * The NVFP4 global scale alone: S = fp32(max|x| / 1536) over x, after the
 * optional rotation ([SS] 2., Escala Global: the per-tensor FP32 scale puts
 * the largest value at the top of the E2M1 x E4M3 range, 6 * 256).  This is
 * the first step of fp4q_quantize_nvfp4, and fp4q_quantize_nvfp4 with
 * FP4Q_GIVEN_SCALE and this S gives bit for bit what one call computing S
 * gives.  Splitting the two serves callers that share one S across several
 * calls: the row shards of one tensor (on one device or several) each
 * compute their S, take the maximum (the rounding is monotone, so that
 * maximum is the S of the whole tensor) and pass it with FP4Q_GIVEN_SCALE.
 *
 *   x, dtype, rows, cols, ld, hadamard_n  as for fp4q_quantize_nvfp4
 *               (cols a multiple of 16 and of hadamard_n).
 *   global_scale [1] float32 S (device, out); 0 for an empty matrix.
 *   workspace   fp4q_workspace_bytes() bytes of device memory.
 *
 * Errors as for fp4q_quantize_nvfp4; a non-finite x sets
 * FP4Q_DATA_NONFINITE_INPUT in the workspace's status word (asynchronous).
 */
fp4q_status_t fp4q_global_scale_nvfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                      int64_t ld, int hadamard_n, float *global_scale, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * MXFP4 quantization with an exponent-window search over E8M0 block scales
 * ([MR] 1., 2.: power-of-two scales, MSE-optimised grid; [TQ] S-step for the
 * base), optionally after a block Hadamard rotation.
 *
 *   block       32.
 *   off_lo, off_hi  window in powers of two around the base exponent,
 *               -16 <= off_lo <= 0 <= off_hi <= 16 (default -1, 0; 0, 0 is
 *               the AbsMax rule).
 *   scales      [rows * cols / 32] E8M0 bytes (E + 127) (out).
 *   block_loss  [rows * cols / 32] float32 loss in the units of x (may be NULL).
 *   offsets     [rows * cols / 32] int8 chosen exponent minus base (may be NULL).
 *   Other arguments as for fp4q_quantize_nvfp4; there is no global scale.
 *
 * Computation: u = |x|; per block E_base = least E with 6 * 2^E >= max u,
 * clamped to [-127, 127]; for E = max(-127, E_base+off_lo) ..
 * min(127, E_base+off_hi): q = E2M1 nearest to fp32(u * 2^-E),
 * e = fp32(u - q*2^E); the loss is the fused in-order sum above over all
 * 32 elements of the block (one rounding per term); the smallest E with the
 * least loss is chosen.
 */
fp4q_status_t fp4q_quantize_mxfp4(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                  int64_t ld, const float *importance, int block, fp4q_loss_t loss,
                                  int off_lo, int off_hi, int hadamard_n, uint8_t *codes,
                                  uint8_t *scales, float *block_loss, int8_t *offsets,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * FOCUS forward quantizer with coupled-relaxation coefficients ([FC]
 * Metodologia 2. CRS and 3. DGS): the codes of sub-block k of a hardware
 * block are Q(x / (S_dq * c_k)), where S_dq is the block's stored
 * dequantization scale and c_k a full-precision FP16 coefficient per
 * sub-block; dequantization keeps using S_dq alone ([FC] 4.).
 *
 *   format      FP4Q_NVFP4 (blocks of 16, E4M3 scale patterns, FP32 global
 *               scale) or FP4Q_MXFP4 (blocks of 32, E8M0 scale bytes).
 *   x, dtype, rows, cols, ld   input matrix as for the quantize calls.
 *   scales      [rows * cols / block] stored scales (e.g. from a quantize call).
 *   global_scale [1] float32 S (NVFP4; ignored for MXFP4, may be NULL).
 *   coeffs      [rows * cols / sub_block] FP16 coefficients, row-major, or
 *               NULL for all ones (then the codes equal the
 *               round-to-nearest codes at the given scales).
 *   sub_block   4, 8 or 16 (NVFP4); 4, 8, 16 or 32 (MXFP4).
 *   codes       [rows * cols / 2] packed codes (out).
 *   dequant_out [rows * cols] float32 x_hat = q * S_dq, dense row-major
 *               (out; may be NULL).
 *   workspace   as for the quantize calls (status word at byte 0).
 *
 * Computation (each float32 step rounded to nearest even): NVFP4 u =
 * fp32(|x| * fp32(1/S)), Vc = fp32(E4M3(p) * c_k); MXFP4 u = |x|,
 * Vc = fp32(2^E * c_k); R = fp32(1/Vc), q = E2M1 nearest to fp32(u * R).
 * A scale pattern outside 1..126 (NVFP4) or 255 (MXFP4), a coefficient
 * that is not finite and positive, or an infinite R sets
 * FP4Q_DATA_BAD_SCALE; non-finite x sets FP4Q_DATA_NONFINITE_INPUT.
 */
fp4q_status_t fp4q_quantize_relaxed(fp4q_format_t format, const void *x, fp4q_dtype_t dtype, int64_t rows,
                                    int64_t cols, int64_t ld, const uint8_t *scales,
                                    const float *global_scale, const uint16_t *coeffs, int sub_block,
                                    uint8_t *codes, float *dequant_out, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * GPTQ with ScaleSweep group scales for NVFP4 ([SS] Principais
 * Contribuições 2: the bounded sweep chooses block scales in GPTQ
 * pipelines too; [MR] 2., MR-GPTQ component 1: the grid is chosen per
 * format).  GPTQ (only named on the pages) is the published column-by-column
 * quantization with error feedback through the inverse Hessian.
 *
 *   w          [rows x cols] float32, leading dimension ld (multiple of 4):
 *              working storage, OVERWRITTEN (on return it holds the scaled
 *              quantization errors).
 *   w_in       [rows x cols] float32, leading dimension ld_in (>= cols,
 *              multiple of 4): the weight, read only; or NULL when w holds
 *              the weight (quantized in place).  With a separate w_in, no
 *              copy of the weight is needed: each column is read from w_in
 *              until an update first writes it into w.  w_in must not
 *              overlap w unless it is w itself.
 *   cols       a multiple of 128 (the lazy-batch width).
 *   hinv_chol  [cols x cols] float32 row-major U, the upper Cholesky factor
 *              of H^-1 (H = X^T X of calibration activations, damped by the
 *              caller), so that H^-1 = U^T U.
 *   importance [cols] float32 per-column WMSE weights, or NULL for MSE.
 *   off_lo, off_hi  E4M3 bit-pattern window of the group-scale search
 *              (at most 16 candidates, off_hi - off_lo <= 15), e.g. -3, 7
 *              (MSE) or -8, 7 (WMSE).
 *   flags      0 or FP4Q_GIVEN_SCALE (read S from *global_scale).
 *   codes, scales, global_scale  as for fp4q_quantize_nvfp4 (no losses);
 *              codes must be 4-byte aligned.
 * Alignment: w and hinv_chol 16-byte aligned, otherwise FP4Q_ERR_ALIGN.
 *
 * Computation: S = fp32(max|w| / 1536) from w before any update.  Columns
 * are processed in order; when column c opens a 16-column group, each row's
 * scale pattern is the sweep's choice on the group's current values;
 * column c is rounded to nearest at that scale, its scaled error
 * err = fp32(fp32(w_c - x_hat_c) * fp32(1 / U[c][c])) is kept, and every
 * later column j of the same 128-column batch becomes fma(-err, U[c][j],
 * w_j).  Later columns receive earlier errors as contractions
 * w -= Err * U[rows of Err, cols] (lazy batches): within each block of 1024
 * columns, after batch t of the block (m the lowest set bit of t + 1) the
 * last m batches' errors reach the next m batches' columns, on fp32 matrix
 * cores; after each block all later columns get the whole block's errors in
 * one contraction on the bf16 matrix cores, each fp32 operand split exactly
 * into three bf16 parts and the six part products down to order 2^-16 kept
 * (the dropped ones at most ~2^-23 of a product).  The float32 grouping of
 * the updates is therefore not that of 128-column batches alone.  A
 * non-positive or non-finite diagonal entry of U sets FP4Q_DATA_BAD_HESSIAN.
 * Argument errors: FP4Q_ERR_SHAPE for ld or ld_in below cols, FP4Q_ERR_ALIGN
 * for w, w_in or hinv_chol not 16-byte aligned or ld, ld_in not multiples
 * of 4.
 */
fp4q_status_t fp4q_gptq_nvfp4(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                              int64_t ld_in, const float *hinv_chol, const float *importance, int off_lo,
                              int off_hi, uint32_t flags, uint8_t *codes, uint8_t *scales,
                              float *global_scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * GPTQ with MXFP4 group scales ([MR] 2., MR-GPTQ component 1: the grid is
 * optimised per format, MXFP4 as well as NVFP4).  The same procedure as
 * fp4q_gptq_nvfp4 with 32-column groups: when column c opens a group, each
 * row's E8M0 exponent is the exponent sweep's choice (fp4q_quantize_mxfp4's
 * search: base exponent, window of exponent offsets, the block loss as one
 * in-order sum over its 32 elements) on the group's current values; column c is rounded at
 * 2^E, x_hat = q * 2^E exactly, and the scaled errors and updates are those
 * of fp4q_gptq_nvfp4.  There is no global scale.
 *
 *   w, rows, cols, ld, w_in, ld_in, hinv_chol, importance  as for
 *              fp4q_gptq_nvfp4.
 *   off_lo, off_hi  exponent window (at most 16 candidates), e.g. -1, 0.
 *   codes      [rows x cols/2] packed E2M1 codes (4-byte aligned).
 *   scales     [rows x cols/32] E8M0 bytes (E + 127).
 *   workspace  fp4q_workspace_bytes() bytes (status word).
 * A non-finite weight sets FP4Q_DATA_NONFINITE_INPUT, a negative or
 * non-finite importance FP4Q_DATA_BAD_IMPORTANCE, a bad diagonal of U
 * FP4Q_DATA_BAD_HESSIAN.  Argument errors as for fp4q_gptq_nvfp4.
 */
fp4q_status_t fp4q_gptq_mxfp4(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                              int64_t ld_in, const float *hinv_chol, const float *importance, int off_lo,
                              int off_hi, uint8_t *codes, uint8_t *scales, void *workspace,
                              size_t workspace_bytes, void *stream);

/*
 * GPTQ with static activation reordering ([MR] 2., MR-GPTQ component 2:
 * GPTQ's column-reordering heuristic is applied once, when quantizing, so
 * that inference shuffles nothing).  The columns are processed in the
 * caller's order perm (GPTQ's heuristic puts the columns with the largest
 * diagonal entries of H first); the groups stay the contiguous blocks of the
 * stored order, and each group's scale is fixed before any update.
 *
 *   w          [rows x cols] float32, leading dimension ld (multiple of 4):
 *              working storage, OVERWRITTEN (on return it holds the scaled
 *              errors in processing order).
 *   w_in       [rows x cols] float32, leading dimension ld_in (>= cols,
 *              multiple of 4): the weight in the stored order, read only;
 *              required, and must not overlap w.
 *   perm       [cols] int32 device array: slot j of the processing order
 *              takes stored column perm[j].
 *   hinv_chol  [cols x cols] float32 row-major U, the upper Cholesky factor
 *              of the inverse of the (damped) Hessian permuted to the
 *              processing order, Hp = H[perm][:, perm], so Hp^-1 = U^T U.
 *   importance [cols] float32 WMSE weights in the stored order (16-byte
 *              aligned), or NULL for MSE.
 *   off_lo, off_hi, flags, global_scale  as for fp4q_gptq_nvfp4.
 *   codes      [rows x cols/2] packed E2M1 codes in the stored order (out;
 *              8-byte aligned).
 *   scales     [rows x cols/16] E4M3 patterns in the stored order (out).
 *   workspace  fp4q_gptq_static_workspace_bytes(rows, cols) bytes (the
 *              status word, the inverse order and the codes in processing
 *              order), 256-byte aligned.
 * Computation: S and every group's scale are those of fp4q_quantize_nvfp4
 * on w_in with the same importance, window and flags (the sweep on the
 * weight before any update).  Slot j is then processed as column j of
 * fp4q_gptq_nvfp4 would be, on the permuted weight with U, except that it
 * is rounded at the scale of its stored group (perm[j] / 16) and no sweep
 * runs at group starts; codes are written back to the stored positions.
 * Data errors: those of fp4q_quantize_nvfp4 and fp4q_gptq_nvfp4, and
 * FP4Q_DATA_BAD_PERM when perm is not a permutation (out-of-range entries
 * are clamped, so nothing is read out of bounds; the results are then
 * meaningless).  Argument errors as for fp4q_gptq_nvfp4, FP4Q_ERR_NULL for
 * a NULL w_in or perm, FP4Q_ERR_ARG when w_in and w overlap,
 * FP4Q_ERR_WORKSPACE for a short or misaligned workspace.
 */
size_t fp4q_gptq_static_workspace_bytes(int64_t rows, int64_t cols);

fp4q_status_t fp4q_gptq_static_nvfp4(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                                     int64_t ld_in, const int32_t *perm, const float *hinv_chol,
                                     const float *importance, int off_lo, int off_hi, uint32_t flags,
                                     uint8_t *codes, uint8_t *scales, float *global_scale, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * fp4q_gptq_static_nvfp4 with MXFP4 groups ([MR] 2., components 1 and 2):
 * every group's E8M0 exponent is that of fp4q_quantize_mxfp4 on w_in with
 * the same importance and exponent window (-16 <= off_lo <= 0 <= off_hi <=
 * 16, at most 16 candidates); slot j is rounded at 2^E of its stored group
 * (perm[j] / 32), with no global scale.  Arguments as for
 * fp4q_gptq_static_nvfp4 without flags and global_scale; scales
 * [rows x cols/32] E8M0 bytes.
 */
fp4q_status_t fp4q_gptq_static_mxfp4(float *w, int64_t rows, int64_t cols, int64_t ld, const float *w_in,
                                     int64_t ld_in, const int32_t *perm, const float *hinv_chol,
                                     const float *importance, int off_lo, int off_hi, uint8_t *codes,
                                     uint8_t *scales, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dequantization (the consumer side: only codes and dequantization scales
 * are stored, [FC] 4.).
 *   NVFP4 (block 16): x_hat = sign * fp32(fp32(q * E4M3(scale)) * S), S read
 *   from global_scale (device).  MXFP4 (block 32): x_hat = sign * q *
 *   2^(scale - 127); global_scale is ignored and may be NULL.
 *   out [rows * cols] float32, dense row-major.
 *   Scale bytes are not checked: 0x7F (E4M3) and 0xFF (E8M0) decode as NaN.
 */
fp4q_status_t fp4q_dequantize(fp4q_format_t format, const uint8_t *codes, const uint8_t *scales,
                              const float *global_scale, int64_t rows, int64_t cols, int block,
                              float *out, void *stream);

/*
 * Block Hadamard rotation ([MR] 2., component 3): each row's groups of n
 * contiguous columns times H_n / sqrt(n), H_n the Sylvester Hadamard matrix
 * in natural order, n in {16, 32, 64, 128}.  Evaluated as a fast transform:
 * stages h = 1, 2, ..., n/2 map (z_i, z_{i+h}) to (z_i + z_{i+h},
 * z_i - z_{i+h}) for i with (i & h) == 0, then every value is multiplied by
 * fp32(1/sqrt(n)).  The transform is its own inverse (up to rounding).
 *   out [rows * cols] float32, dense row-major.  Inf/NaN propagate.
 */
fp4q_status_t fp4q_block_hadamard(const void *x, fp4q_dtype_t dtype, int64_t rows, int64_t cols,
                                  int64_t ld, int n, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_H */
