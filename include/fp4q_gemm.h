/* fp4q_gemm.h -- W4A4 matrix products of microscaled FP4 operands on gfx950.
 *
 * Consumer of the quantizers in fp4q.h.  "Bridging the Gap Between Promise
 * and Performance for Microscaling FP4 Quantization" (2. Metodologia;
 * 3. QuTLASS): weights and activations are both quantized to FP4 (W4A4),
 * and their product runs on FP4 matrix hardware.  With a block rotation,
 * both operands carry the same block Hadamard along K, and it cancels in the
 * product (H H^T = I; the same page, 2., micro-rotation).  Quantizing A and
 * B with fp4q_quantize_mxfp4(..., hadamard_n = n, ...) therefore gives the
 * product of the unrotated matrices, up to quantization error.
 *
 * All pointers are device pointers; stream is a hipStream_t (NULL = the
 * default stream).  The call enqueues its kernels (one to three) and
 * returns.  It allocates nothing and keeps no state.  Argument errors are returned synchronously,
 * before anything is enqueued.
 */
#ifndef FP4Q_GEMM_H
#define FP4Q_GEMM_H

#include <stddef.h>
#include <stdint.h>

#include "fp4q.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C = alpha * A_hat * B_hat^T for MXFP4 operands.
 *
 *   a_codes   [m x k/2] bytes, row-major, row stride k/2: the E2M1 codes of
 *             A (activations, one row per token).  Element 2i of a row is in
 *             the low nibble of byte i, and bit 3 of a nibble is the sign.
 *             This is the layout fp4q_quantize_mxfp4 writes.
 *   a_scales  [m x k/32] E8M0 bytes, row-major: element k of row r is
 *             q * 2^(a_scales[r][k/32] - 127).  Byte 255 encodes NaN.
 *   b_codes, b_scales  the same for B [n x k] (weights, one row per output
 *             channel).
 *   m, n, k   m, n >= 0; k > 0 and a multiple of 32.
 *   alpha     float32 factor applied to the float32 accumulator.
 *   out_dtype FP4Q_F32 or FP4Q_BF16 (round to nearest even).
 *   c         [m x n] row-major with leading dimension ldc >= n (elements),
 *             written in full.  It must not overlap the inputs.
 *   workspace optional device memory (NULL for none) of at least
 *             fp4q_gemm_mxfp4_workspace_bytes(m, n, k) bytes, 16-byte
 *             aligned; its contents are overwritten.  It is used when K is
 *             a multiple of 256:
 *             - products large enough for 256 x 256 tiles on every CU first
 *               copy both operands' scales there in a stage-major order
 *               ([k/256][rows][8 bytes]), and then load each stage's scales
 *               in 1 KB pieces (the MR-GPTQ page, 3.: QuTLASS reorganises
 *               scales for its FP4 product).  The result is identical to
 *               the one without a workspace;
 *             - few-token products (m <= 64) whose column tiles alone would
 *               leave CUs idle, and that the few-token kernel below does not
 *               take, split K into S contiguous ranges (S chosen from m, n
 *               and k) and keep the S float32 partial sums there.
 *
 * Arithmetic: the products of two decoded elements are exact.  They are
 * summed on the matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4), 64
 * elements of K per step, each step added to a float32 accumulator.  When K
 * is a multiple of 128, K is walked in stages of 256 elements (128 when K is
 * not a multiple of 256), stages in ascending order, and step j of a stage
 * holds its 32-element blocks j and j + 4 (j and j + 2 for 128-element
 * stages); otherwise step j holds elements 64 j .. 64 j + 63.  With a K
 * split, each range is summed that way and
 * the S partial sums are then added in ascending K order, which can round
 * differently from a single accumulation.  Products of at most 16 tokens
 * with K a multiple of 512 and at most 16384 (and of at most 64 tokens with
 * n <= 4096 and K at most 8192), with both scale arrays 16-byte aligned, go
 * to a few-token kernel (no workspace) that sums on
 * v_mfma_scale_f32_16x16x128_f8f6f4: K is cut into W contiguous ranges of S
 * steps of 128 contiguous elements (S = 4 or 8, W = k / (128 S) <= 16),
 * each range is accumulated step by step in float32, and the W range sums
 * are added in ascending K order.  Either way the result differs from the
 * exact product by a few float32 roundings per step.
 *
 * Alignment: a_codes and b_codes 16-byte aligned.  c aligned to its element
 * size.
 *
 * Returns FP4Q_ERR_NULL for a missing pointer (none is needed when m or n
 * is 0), FP4Q_ERR_SHAPE for a bad m, n, k or ldc, FP4Q_ERR_ARG for an
 * unknown out_dtype, FP4Q_ERR_WORKSPACE for a workspace smaller than
 * fp4q_gemm_mxfp4_workspace_bytes, FP4Q_ERR_ALIGN, or FP4Q_ERR_HIP if the
 * launch fails.
 */
fp4q_status_t fp4q_gemm_mxfp4(const uint8_t *a_codes, const uint8_t *a_scales, const uint8_t *b_codes,
                              const uint8_t *b_scales, int64_t m, int64_t n, int64_t k, float alpha,
                              fp4q_dtype_t out_dtype, void *c, int64_t ldc, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Workspace that speeds up fp4q_gemm_mxfp4 when K is a multiple of 256: the
 * larger of (m + n) * k / 32 + 32 bytes (scale copies) and, for a split few-
 * token product, S * m * n * 4 bytes (partial sums; sized also where the
 * few-token kernel, which needs none, takes the product).  0 when K is not a
 * multiple of 256 (no workspace is used) and for invalid sizes. */
size_t fp4q_gemm_mxfp4_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Workspace the NVFP4 product needs: (m + n) * roundup(k, 32) * 2 bytes (the
 * operands decoded to bfloat16); for the few-token products (above), which
 * decode in registers, 0 or KS * m * n * 4 bytes (their K segments' partial
 * sums); 0 for invalid sizes. */
size_t fp4q_gemm_nvfp4_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* C = fp32(S_a * S_b) * (A_hat * B_hat^T) for NVFP4 operands, where A_hat and
 * B_hat hold q * E4M3(p) without the global scales.
 *
 * The NVFP4 tensors are the ones "Resumo Tecnico: ScaleSweep" describes:
 * E2M1 codes, one E4M3 scale per 16 elements of K, and one FP32 global scale
 * per tensor.  This is the layout fp4q_quantize_nvfp4 writes.
 *   a_codes   [m x k/2] bytes, row-major (element 2i in the low nibble of
 *             byte i; bit 3 of a nibble is the sign).
 *   a_scales  [m x k/16] E4M3 bytes (bit 7 sign; 0x7F / 0xFF NaN).
 *   a_global  device pointer to A's float32 global scale S_a.
 *   b_codes, b_scales, b_global  the same for B [n x k].
 *   m, n, k   m, n >= 0; k > 0 and a multiple of 16.
 *   out_dtype, c, ldc  as for fp4q_gemm_mxfp4.
 *   workspace device memory of at least fp4q_gemm_nvfp4_workspace_bytes(m,
 *             n, k) bytes, 16-byte aligned; its contents are overwritten.
 *             None is needed (NULL is accepted) where that size is 0 (most
 *             few-token products below).
 *
 * The scaled FP4 matrix core takes only power-of-two (E8M0) scales per 32
 * elements.  Folding an E4M3 block scale into the elements would need
 * up to 6 significant bits per element, more than an 8-bit float holds.
 * So each element is decoded to q * E4M3(p), which bfloat16 holds exactly.
 * That costs one pass over both operands into the workspace.  The products
 * run on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16), where each
 * product is exact, summed in float32 one 16-element step of K at a time in
 * ascending K order.  The result is multiplied by fp32(S_a * S_b).
 *
 * Products with K a multiple of 128 that are too small for 256 x 256 tiles
 * on every CU (and have 16-byte aligned codes, 4-byte aligned scales) skip
 * that pass as well: the codes are staged in LDS and decoded in registers
 * to float16, which holds q * E4M3(p) exactly too, and summed on
 * v_mfma_f32_32x32x16_f16.  K moves in stages of 128 elements, ascending;
 * step s = 0 .. 7 of a stage holds its elements 8 s .. 8 s + 7 and
 * 64 + 8 s .. 64 + 8 s + 7, steps ascending.  The workspace is not touched.
 *
 * Products of at most 32 tokens (64 on outputs of at most 4096 columns)
 * with K a multiple of 256 skip that pass too, in a few-token kernel that
 * decodes in registers and sums on v_mfma_f32_16x16x32_f16, when K fits its
 * register budget: k / 128 groups over at most 16 waves of S groups each
 * (S = 2, 4 or 8, S ceil(m / 16) <= 8), and over KS = 1, 2 or 4 workgroups
 * per column tile (each writing its segment's float32 sums to the
 * workspace; the workspace query sizes them).  K is thus cut into KS W
 * contiguous ranges of S groups of 128 elements; each range is accumulated
 * in float32 one 32-element step at a time, and the range sums are added in
 * ascending K order before the multiplication by fp32(S_a * S_b).
 *
 * Alignment: a_codes and b_codes 8-byte aligned (16-byte, and the scale
 * arrays too, for the few-token products); the global-scale pointers 4-byte
 * aligned; c aligned to its element size.
 *
 * Returns FP4Q_ERR_NULL, FP4Q_ERR_SHAPE, FP4Q_ERR_ARG, FP4Q_ERR_WORKSPACE,
 * FP4Q_ERR_ALIGN or FP4Q_ERR_HIP, as for fp4q_gemm_mxfp4 (nothing is needed
 * when m or n is 0).
 */
fp4q_status_t fp4q_gemm_nvfp4(const uint8_t *a_codes, const uint8_t *a_scales, const float *a_global,
                              const uint8_t *b_codes, const uint8_t *b_scales, const float *b_global, int64_t m,
                              int64_t n, int64_t k, fp4q_dtype_t out_dtype, void *c, int64_t ldc, void *workspace,
                              size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_GEMM_H */
