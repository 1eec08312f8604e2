/*
 * nf4ref.h - CPU oracle for blockwise NF4 quantization with double quantization.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, plain reference that the
 * GPU library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header, table or
 * constant generator with the GPU library, and it includes nothing from it.
 *
 * Sources (web pages), cited by title and section:
 *   [MF]  "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization,
 *          Double Quantization, and Paged Optimizers" (llms.blog)
 *   [L15] "Lesson 15. NF4 and Double Quantisation" (tokencemetery)
 *   [QP]  "QLoRA in Production: 4-bit NormalFloat & Double Quantization Deep
 *          Dive" (devtechtools.org)
 *
 * Fixed parameters: block size B1 = 64 ([MF] "Block-Wise Quantization
 * Mechanics"), double-quantization block B2 = 256 ([MF] "Double Quantization").
 *
 * Layout conventions (the pages leave them open; they are readings, not pins):
 *   - codes: two 4-bit codes per byte, element 2j in the low nibble, element
 *     2j+1 in the high nibble; for odd n the last high nibble is 0.
 *     PARITY UNPINNED (a storage convention the pages do not fix).
 *   - blocks are consecutive runs of 64 elements of the flattened tensor; the
 *     last block may be partial and takes the max over its valid elements.
 *
 * All functions return 0 on success and a negative value on invalid input
 * (NULL pointer, negative size, non-finite input).
 */
#ifndef NF4REF_H
#define NF4REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NF4REF_BLOCK 64
#define NF4REF_DQ_BLOCK 256

enum { NF4REF_F32 = 0, NF4REF_BF16 = 1 };

/* The 16 NF4 levels exactly as printed in [MF] "4-Bit NormalFloat (NF4)". */
void nf4ref_codebook(float q[16]);

/* Standard normal quantile (inverse CDF) by bisection on 0.5*erfc(-x/sqrt 2). */
double nf4ref_normal_quantile(double p);

/* The asymmetric quantile construction of [MF] "4-Bit NormalFloat (NF4)":
 * 8 positive levels from probabilities evenly spaced from delta down to 1/2,
 * 7 negative levels likewise, an exact zero, all divided by the largest.
 * Writes 16 ascending levels. */
int nf4ref_construct_codebook(double delta, double out[16]);

/* Solves the tail probability delta for which the construction's level 14
 * equals `level14` (bisection on [0.9, 0.9999]). */
double nf4ref_solve_delta(double level14);

/* Nearest-level code of one normalised value n: the first index i that
 * minimises |fl32(n - q_i)| ([MF] "Block-Wise Quantization Mechanics", argmin). */
int nf4ref_nearest_code(float n);
int nf4ref_nearest_code_array(const float *n, int64_t count, uint8_t *out);

/* bf16 <-> fp32. Widening is exact; narrowing rounds to nearest, ties to even. */
float nf4ref_bf16_to_f32(uint16_t h);
uint16_t nf4ref_f32_to_bf16(float f);
int nf4ref_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out);

/* Blockwise NF4 quantization of n elements (dtype NF4REF_F32 or NF4REF_BF16).
 * codes: ceil(n/2) bytes. absmax: ceil(n/64) floats. */
int nf4ref_quantize(const void *w, int dtype, int64_t n, uint8_t *codes, float *absmax);

/* OCP FP8 E4M3FN encode / decode (double-quantization code format). */
uint8_t nf4ref_e4m3_encode(float r);
float nf4ref_e4m3_decode(uint8_t c);
int nf4ref_e4m3_encode_array(const float *r, int64_t n, uint8_t *out);

/* Double quantization of nblocks fp32 absmax values. q: nblocks bytes.
 * scale: ceil(nblocks/256) floats. */
int nf4ref_double_quantize(const float *absmax, int64_t nblocks, uint8_t *q, float *scale);

/* Reconstructed first-level scale of block b: absmax[b] when q == NULL, else
 * fl32(decode(q[b]) * scale[b/256]). */
float nf4ref_block_scale(int64_t b, const float *absmax, const uint8_t *q, const float *scale);

/* Dequantization to fp32 (out_dtype NF4REF_F32) or bf16 (NF4REF_BF16).
 * Uses absmax when q == NULL, else (q, scale). */
int nf4ref_dequantize(const uint8_t *codes, int64_t n, const float *absmax, const uint8_t *q,
                      const float *scale, void *out, int out_dtype);

/* Dequantization of elements [start, start + count) of an n-element tensor,
 * with the block and group indices of the whole tensor. out: count values. */
int nf4ref_dequantize_range(const uint8_t *codes, int64_t n, int64_t start, int64_t count,
                            const float *absmax, const uint8_t *q, const float *scale, void *out,
                            int out_dtype);

/* Storage bytes of an n-element NF4 tensor: codes + scales (dq != 0: 8-bit
 * codes plus fp32 second-level scales; dq == 0: fp32 absmax). */
int64_t nf4ref_storage_bytes(int64_t n, int dq);

/* Forward of the QLoRA linear ([MF] "Forward Pass Computation") on selected
 * rows and columns, in double with no intermediate rounding:
 *   out[i][j] = sum_k x[rows[i],k] * wdeq[cols[j],k]
 *             + s * sum_t (sum_k x[rows[i],k] * A[k,t]) * B[t,cols[j]]
 * x: bf16 [m x K]; wdeq: fp32 [N x K] (the dequantized weight, stored
 * [d_out x d_in]); A: bf16 [K x r]; B: bf16 [r x N]; A == NULL or r == 0
 * skips the adapter. rows/cols may be NULL (all). out: double [nrows x ncols]. */
int nf4ref_linear_forward(const uint16_t *x, int64_t m, int64_t K, int64_t N, const float *wdeq,
                          const uint16_t *A, const uint16_t *B, int32_t r, double s,
                          const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                          double *out);

/* Input gradient ([MF] "Gradient Computation", the activation-gradient
 * equation) on selected rows and columns, in double:
 *   out[i][j] = sum_n dy[rows[i],n] * wdeq[n,cols[j]]
 *             + s * sum_t (sum_n dy[rows[i],n] * B[t,n]) * A[cols[j],t]
 * dy: bf16 [m x N]. out: double [nrows x ncols]. */
int nf4ref_linear_backward_input(const uint16_t *dy, int64_t m, int64_t K, int64_t N,
                                 const float *wdeq, const uint16_t *A, const uint16_t *B,
                                 int32_t r, double s, const int64_t *rows, int64_t nrows,
                                 const int64_t *cols, int64_t ncols, double *out);

/* Gradients of the adapter ([MF] "Gradient Computation", the two adapter
 * equations), in double with no intermediate rounding:
 *   dA = s * X^T (dY B^T)     [K x r]   (the gradient of L1 = A)
 *   dB = s * (X A)^T dY       [r x N]   (the gradient of L2 = B)
 * x: bf16 [m x K]; dy: bf16 [m x N]; A: bf16 [K x r]; B: bf16 [r x N].
 * a_rows (na indices into K) selects the rows of dA, b_cols (nb indices into
 * N) the columns of dB; NULL means all. da: double [na x r] (may be NULL),
 * db: double [r x nb] (may be NULL). Returns 0, or -1 on invalid arguments. */
int nf4ref_lora_grads(const uint16_t *x, const uint16_t *dy, int64_t m, int64_t K, int64_t N,
                      const uint16_t *A, const uint16_t *B, int32_t r, double s,
                      const int64_t *a_rows, int64_t na, double *da, const int64_t *b_cols,
                      int64_t nb, double *db);

/* ---- Variants of the storage format ([MF] "Block-Wise Quantization
 * Mechanics": 64 is the typical block size, so B1 is a parameter; [MF]
 * "Double Quantization (DQ)": the 8-bit float format of the second step is
 * not named, and the step's prose mentions an asymmetric bias / mean
 * subtraction). Readings:
 *   - B1 (blocksize) and B2 (dq_blocksize) are powers of two, B1 in
 *     [16, 4096], B2 in [1, 4096];
 *   - dq_format: NF4REF_DQ_E4M3 (OCP E4M3FN of c1/c2, the default),
 *     NF4REF_DQ_E5M2 (OCP E5M2 of c1/c2, round to nearest even), or
 *     NF4REF_DQ_LINEAR8 (a uniform integer code: the stored group value is the
 *     step u = fl32(c2 / L) with L = 255, or 127 for signed codes; the code is
 *     the nearest integer to fl32(c1 / u), clamped to [0, L] (or [-L, L]);
 *     the scale is reconstructed as fl32(code * u));
 *   - mean offset: mu = fl32(S / fl32(nblocks)), S the pairwise sum of all
 *     c1 of the tensor (nf4ref_pairwise_sum); double quantization then acts on
 *     x = fl32(c1 - mu): c2 = max |x| over the group, the code is the signed
 *     code of fl32(x / c2) (or of fl32(x / u)), and the reconstructed scale is
 *     fl32(fl32(decode * c2) + mu). One fp32 mu per tensor, so the
 *     per-parameter footprint is unchanged. */
enum { NF4REF_DQ_E4M3 = 0, NF4REF_DQ_E5M2 = 1, NF4REF_DQ_LINEAR8 = 2 };

/* nf4ref_quantize with block size B1. absmax: ceil(n/B1) floats. */
int nf4ref_quantize_bs(const void *w, int dtype, int64_t n, int32_t blocksize, uint8_t *codes,
                       float *absmax);

/* OCP FP8 E5M2 encode (round to nearest even; beyond the largest finite value
 * saturates to it) / decode. */
uint8_t nf4ref_e5m2_encode(float r);
float nf4ref_e5m2_decode(uint8_t c);
int nf4ref_e5m2_encode_array(const float *r, int64_t n, uint8_t *out);

/* Pairwise sum in fp32: the values padded with zeros to a power-of-two
 * count, then adjacent pairs added level by level until one value remains. */
float nf4ref_pairwise_sum(const float *x, int64_t n);

/* Double quantization with a block B2, a code format and an optional mean
 * offset (see above). q: nblocks bytes; scale: ceil(nblocks/B2) floats (c2, or
 * the step u for NF4REF_DQ_LINEAR8); offset: one float, written iff
 * mean_offset (may be NULL otherwise). */
int nf4ref_double_quantize_ex(const float *absmax, int64_t nblocks, int32_t dq_blocksize,
                              int dq_format, int mean_offset, uint8_t *q, float *scale,
                              float *offset);

/* The reconstructed scale of block b under the variant; offset == NULL means
 * no mean offset, q == NULL means no double quantization (absmax[b]). */
float nf4ref_block_scale_ex(int64_t b, int32_t dq_blocksize, int dq_format, const float *absmax,
                            const uint8_t *q, const float *scale, const float *offset);

/* nf4ref_dequantize_range with block size B1 and the DQ variant. */
int nf4ref_dequantize_range_ex(const uint8_t *codes, int64_t n, int64_t start, int64_t count,
                               int32_t blocksize, int32_t dq_blocksize, int dq_format,
                               const float *absmax, const uint8_t *q, const float *scale,
                               const float *offset, void *out, int out_dtype);

/* ---- Merging the adapter into the quantized base ([QP] "Step 4: Merging and
 * Inference"; "QLoRA: quantising the part you are not training" (addaly),
 * "What it costs", item 3: a merge into the quantized base must re-quantize).
 * With Y = X W'^T + s (X A) B, the merged weight is
 *   Wm[n][k] = fl32(W'[n][k] + fl32(s * fl32(d[n][k]))),  d[n][k] = sum_j A[k][j] B[j][n]
 * with d summed in double (every product of two bf16 values is exact) and
 * rounded once to fp32, and W' the fp32 dequantized base. The
 * merged weight is then re-quantized blockwise (and double-quantized) as by
 * nf4ref_quantize / nf4ref_double_quantize.
 *   codes, q, scale, absmax: the base ([N x K], q == NULL: plain absmax)
 *   A bf16 [K x r], B bf16 [r x N], s = alpha / r
 *   rows (nrows indices into N, NULL = all): the rows written to wm, fp32
 *   [nrows x K]. Returns 0, or -1 on invalid arguments. */
int nf4ref_merged_weight(const uint8_t *codes, const float *absmax, const uint8_t *q,
                         const float *scale, int64_t N, int64_t K, const uint16_t *A,
                         const uint16_t *B, int32_t r, float s, const int64_t *rows,
                         int64_t nrows, float *wm);

/* ---- Codebook swaps ([MF] "Empirical Performance and Architectural
 * Guidelines", finding 2: NF4 against 4-bit floating point (FP4) and 4-bit
 * integer (Int4); [QP] "1. 4-bit NormalFloat (NF4)", the numpy comparison's
 * naive uniform 4-bit quantizer). The same blockwise scheme with
 * another set of 16 levels in [-1, 1]:
 *   NF4REF_CB_NF4   the printed NF4 list
 *   NF4REF_CB_FP4   OCP FP4 (E2M1) in its own encoding, each value divided by
 *                   6 (fl32(v / 6)): code = 8 * sign + the index of the
 *                   magnitude in {0, .5, 1, 1.5, 2, 3, 4, 6}, so +0 is code 0
 *                   and -0 code 8 (equal to code 0, so the tie rule never
 *                   picks it). The pages name FP4 without defining it; the
 *                   OCP Microscaling Formats specification fixes the encoding.
 *   NF4REF_CB_INT4  16 evenly spaced levels fl32((2k - 15) / 15), k = 0..15:
 *                   the dequantized values (k' + 1/2) / 7.5, k' = -8..7, of the
 *                   uniform toy
 * A block with c1 == 0 gets the code of the level nearest 0. */
enum { NF4REF_CB_NF4 = 0, NF4REF_CB_FP4 = 1, NF4REF_CB_INT4 = 2 };

int nf4ref_codebook_levels(int codebook, float q[16]);

/* nf4ref_quantize_bs with the codebook's levels. */
int nf4ref_quantize_cb(const void *w, int dtype, int64_t n, int32_t blocksize, int codebook,
                       uint8_t *codes, float *absmax);

/* nf4ref_dequantize_range_ex with the codebook's levels. */
int nf4ref_dequantize_range_cb(const uint8_t *codes, int64_t n, int64_t start, int64_t count,
                               int32_t blocksize, int32_t dq_blocksize, int dq_format, int codebook,
                               const float *absmax, const uint8_t *q, const float *scale,
                               const float *offset, void *out, int out_dtype);

/* Storage bytes of an n-element tensor in a variant format: ceil(n/2) code
 * bytes, then either fp32 absmax (dq == 0: 4 per block of B1) or one 8-bit
 * code per block, one fp32 per group of B2 blocks and, with the mean offset,
 * one fp32 for the tensor ([MF] "Double Quantization (DQ)", the footprint
 * with B1 and B2 as parameters). Returns -1 for invalid arguments. */
int64_t nf4ref_storage_bytes_ex(int64_t n, int32_t blocksize, int32_t dq_blocksize, int dq,
                                int mean_offset);

#ifdef __cplusplus
}
#endif
#endif
