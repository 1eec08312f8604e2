/*
 * nf4.h - C ABI of the MI355X (gfx950) NF4 library: blockwise 4-bit
 * NormalFloat quantization with double quantization of the block scales,
 * dequantization, and the fused NF4-dequant linear (forward and input
 * gradient) with the low-rank adapter side path.
 *
 * Sources (web pages), cited by title and section:
 *   [MF]  "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization,
 *          Double Quantization, and Paged Optimizers" (llms.blog)
 *   [L15] "Lesson 15. NF4 and Double Quantisation" (tokencemetery)
 *   [QP]  "QLoRA in Production: 4-bit NormalFloat & Double Quantization Deep
 *          Dive" (devtechtools.org)
 *
 * Conventions shared by every entry point:
 *   - Every buffer is allocated and owned by the caller. Buffers marked
 *     "device" must be device memory of the current HIP device; the library
 *     keeps no pointer after a call returns and allocates nothing.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; the host is never synchronised.
 *     Results are valid in stream order after the call.
 *   - Arguments are validated on the host before any HIP call. On an error the
 *     call returns a non-zero nf4_status and launches nothing. NF4_ERR_LAUNCH
 *     is returned when the HIP runtime reports a launch failure.
 *   - A size of zero elements (n == 0, m == 0) returns NF4_OK and launches nothing.
 *   - Alignment: element buffers (weights, codes, activations, outputs, the
 *     workspace) must be 16-byte aligned; scale buffers (absmax, absmax_q,
 *     absmax_scale) must be 4-byte aligned. Otherwise NF4_ERR_ALIGN.
 *   - Only block size 64 ([MF] "Block-Wise Quantization Mechanics", B1 = 64)
 *     and double-quantization block 256 ([MF] "Double Quantization (DQ)",
 *     B2 = 256) are supported; anything else is NF4_ERR_UNSUPPORTED.
 *   - Non-finite inputs are outside the contract (their output is unspecified).
 *
 * Packed storage layout of an n-element tensor (row-major flattening):
 *   codes          uint8[ceil(n/2)]    element 2j in the low nibble of byte j,
 *                                      element 2j+1 in the high nibble; for odd
 *                                      n the final high nibble is 0
 *   absmax         float[ceil(n/64)]   c1 of each 64-element block
 *   absmax_q       uint8[ceil(n/64)]   E4M3FN code of c1/c2 (double quantization)
 *   absmax_scale   float[ceil(ceil(n/64)/256)]  c2 of each group of 256 blocks
 * The last block / group may be partial; it covers the remaining elements.
 */
#ifndef NF4_H
#define NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NF4_OK = 0,
    NF4_ERR_NULL = 1,        /* a required pointer is NULL */
    NF4_ERR_SIZE = 2,        /* negative size, K % 64 != 0, r out of range, too large */
    NF4_ERR_UNSUPPORTED = 3, /* block size, DQ block size, dtype or format not supported */
    NF4_ERR_ALIGN = 4,       /* a buffer is not aligned as required */
    NF4_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than nf4_linear_workspace_size */
    NF4_ERR_LAUNCH = 6       /* the HIP runtime reported an error at launch */
} nf4_status;

/* Element types. Entry points take them as int32_t (an nf4_dtype value), so
 * that any value a caller passes is representable and an unknown one is
 * rejected with NF4_ERR_UNSUPPORTED. */
typedef enum { NF4_F32 = 0, NF4_BF16 = 1 } nf4_dtype;

/* Human-readable name of a status code (static string). */
const char *nf4_status_string(int status);

/* The 16 NF4 levels q_0..q_15 used by every kernel: the values printed in [MF]
 * "4-Bit NormalFloat (NF4)". Returns a pointer to a static host array. */
const float *nf4_codebook(void);

/* Bytes of the packed storage of an n-element tensor: codes plus either fp32
 * absmax (double_quant == 0) or 8-bit codes plus fp32 second-level scales.
 * ([L15] "Double quantisation": 0.5625 and ~0.5159 bytes per parameter.)
 * Returns -1 for n < 0 or unsupported block sizes. */
int64_t nf4_storage_bytes(int64_t n, int32_t blocksize, int32_t dq_blocksize, int32_t double_quant);

/* Blockwise NF4 quantization ([MF] "Block-Wise Quantization Mechanics"), with
 * the double quantization of the block scales fused in
 * ([MF] "Double Quantization (DQ)").
 *   w             device, n elements, fp32 or bf16 (w_dtype), 16-byte aligned
 *   codes         device out, ceil(n/2) bytes
 *   absmax        device out or NULL, ceil(n/64) floats: c1 = max |w| per block
 *   absmax_q      device out or NULL, ceil(n/64) bytes: E4M3FN(c1 / c2)
 *   absmax_scale  device out or NULL, one float per 256 blocks: c2 = max c1
 * absmax_q and absmax_scale are both given (double quantization) or both NULL
 * (then absmax is required). For each element the code is the index of the
 * nearest level to fl32(w / c1), lower index on an exact tie; a block with
 * c1 == 0 gets code 7 (the zero level); a group with c2 == 0 gets code8 0. */
nf4_status nf4_quantize(const void *w, int32_t w_dtype, int64_t n, int32_t blocksize,
                        uint8_t *codes, float *absmax, int32_t dq_blocksize, uint8_t *absmax_q,
                        float *absmax_scale, void *stream);

/* Double quantization of existing fp32 block scales ([MF] "Double
 * Quantization (DQ)"): c2 = max over each group of 256 of |absmax|, and
 * absmax_q[b] = E4M3FN(fl32(absmax[b] / c2)) with round to nearest even
 * (0 when c2 == 0). Block absmax values are >= 0; a negative value is
 * encoded with the E4M3 sign bit (bit 7 on the magnitude's code), as the
 * format defines. Every absmax value must be finite: NaN or infinity is
 * outside the contract (the result is unspecified; nothing faults).
 *   absmax        device, nblocks floats;  absmax_q device out, nblocks bytes;
 *   absmax_scale  device out, ceil(nblocks/256) floats. */
nf4_status nf4_double_quantize(const float *absmax, int64_t nblocks, int32_t dq_blocksize,
                               uint8_t *absmax_q, float *absmax_scale, void *stream);

/* Dequantization ([MF] "Block-Wise Quantization Mechanics", reconstruction;
 * the dequantize(c1^FP8, c2, W^NF4) of "Forward Pass Computation"):
 *   scale(b) = absmax[b]                                  if absmax_q == NULL
 *            = fl32(decodeE4M3(absmax_q[b]) * absmax_scale[b/256])  otherwise
 *   out[i]   = fl32(q[code_i] * scale(i/64)), rounded to nearest-even bf16
 *              when out_dtype == NF4_BF16.
 *   codes device ceil(n/2) bytes; out device n elements (16-byte aligned). */
nf4_status nf4_dequantize(const uint8_t *codes, int64_t n, int32_t blocksize, const float *absmax,
                          const uint8_t *absmax_q, const float *absmax_scale,
                          int32_t dq_blocksize, void *out, int32_t out_dtype, void *stream);

/* One tensor of a batched call: the buffers that nf4_quantize and
 * nf4_dequantize take for an n-element tensor (block size 64, DQ block 256),
 * with the same layout, alignment and NULL rules.
 *   w             device, n elements of the call's dtype: the input of
 *                 nf4_quantize_batched, the output of nf4_dequantize_batched
 *                 (16-byte aligned)
 *   n             elements, >= 0 (an entry with n == 0 is skipped)
 *   codes         device, ceil(n/2) bytes (16-byte aligned)
 *   absmax        device or NULL, ceil(n/64) floats
 *   absmax_q      device or NULL, ceil(n/64) bytes
 *   absmax_scale  device or NULL, ceil(n/16384) floats
 * absmax_q and absmax_scale are both set (double quantization) or both NULL
 * (then absmax is required), per entry. */
typedef struct {
    void *w;
    int64_t n;
    uint8_t *codes;
    float *absmax;
    uint8_t *absmax_q;
    float *absmax_scale;
} nf4_batch_entry;

/* nf4_quantize of each of `count` tensors, e.g. every weight of a model
 * ([MF] "Block-Wise Quantization Mechanics" and "Double Quantization (DQ)",
 * applied per tensor). Each entry's outputs are exactly those of
 * nf4_quantize(e.w, w_dtype, e.n, 64, e.codes, e.absmax, 256, e.absmax_q,
 * e.absmax_scale, stream). The full 16384-weight groups of up to 32 entries
 * share one launch, and the partial last groups of up to 32 entries another,
 * so small tensors do not each pay a launch's ramp-up and drain.
 *   entries  host array of count entries, read during the call only
 *   count    >= 0
 * Every entry is validated before anything is launched; the first invalid
 * entry decides the status. Outputs of different entries must not overlap. */
nf4_status nf4_quantize_batched(const nf4_batch_entry *entries, int32_t count, int32_t w_dtype,
                                void *stream);

/* nf4_dequantize of each of `count` tensors, batched the same way: entry e's
 * w receives nf4_dequantize(e.codes, e.n, 64, e.absmax, e.absmax_q,
 * e.absmax_scale, 256, e.w, out_dtype, stream). */
nf4_status nf4_dequantize_batched(const nf4_batch_entry *entries, int32_t count,
                                  int32_t out_dtype, void *stream);

/* A frozen NF4 weight W stored [n_out x k_in] row-major (d_out x d_in, the
 * transpose of [MF]'s W in R^{d_in x d_out}), quantized with nf4_quantize over
 * its flattening. Either absmax_q + absmax_scale (double quantization) or
 * absmax must be set. k_in must be a multiple of 64 so that no block crosses
 * a row; groups of 256 blocks may cross rows. */
typedef struct {
    const uint8_t *codes;
    const uint8_t *absmax_q;
    const float *absmax_scale;
    const float *absmax;
    int64_t n_out; /* N = d_out */
    int64_t k_in;  /* K = d_in  */
    int32_t blocksize;
    int32_t dq_blocksize;
} nf4_weight;

/* Bytes of device workspace that nf4_linear_forward / nf4_linear_backward_input
 * need for m rows and adapter rank r (0 when r == 0): with rp = r rounded up
 * to 64, the bf16 adapter product [m x rp] rounded up to 256 bytes, followed
 * by 8 fp32 partial sums of it ([8 x m x rp], the split-K staging of the
 * adapter's down-projection). */
size_t nf4_linear_workspace_size(int64_t m, int32_t r);

/* Fused QLoRA linear forward ([MF] "Forward Pass Computation"):
 *   Y = X . dequantize(W)^T + lora_scale * (X . A) . B
 *   x        device bf16 [m x K] row-major
 *   lora_a   device bf16 [K x r] row-major, or NULL (no adapter; then r must be 0)
 *   lora_b   device bf16 [r x N] row-major
 *   y        device bf16 [m x N] out
 * bf16 operands, fp32 accumulation, bf16 output. lora_scale is alpha/r.
 * 0 <= r <= 256. workspace: device, >= nf4_linear_workspace_size(m, r) bytes
 * (holds the bf16 product X.A); may be NULL when r == 0. */
nf4_status nf4_linear_forward(const void *x, int64_t m, const nf4_weight *w, const void *lora_a,
                              const void *lora_b, int32_t r, float lora_scale, void *y,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the device scratch array that nf4_linear_forward_noalloc uses in
 * place of a workspace (32 MiB; held on each GPU the library runs on until the
 * process ends). */
#define NF4_NOALLOC_SCRATCH_BYTES (32u << 20)

/* nf4_linear_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. It computes exactly what nf4_linear_forward computes (the same
 * kernels, in the same order, so the same bits), with the same arguments less
 * the workspace, which comes from a static device array of
 * NF4_NOALLOC_SCRATCH_BYTES per GPU instead. The call allocates nothing and
 * calls no allocating routine. The caller still owns x, the adapter and y.
 *   Limit: nf4_linear_workspace_size(m, r) <= NF4_NOALLOC_SCRATCH_BYTES, else
 *          NF4_ERR_SIZE, nothing launched (about m * r <= 986,000 after r is
 *          rounded up to 64: m = 4096 takes r up to 192).
 *   The scratch of a GPU is shared by every call on it and keeps the last
 *   call's contents; nothing in it has to start at zero (each call writes
 *   every byte it reads). Calls that overlap on one GPU (different streams,
 *   or host threads) race on it: order them on one stream.
 *   The stream must belong to the current device. The first call on a device
 *   looks up that device's copy of the array (hipGetSymbolAddress); if that
 *   fails the call returns NF4_ERR_LAUNCH. */
nf4_status nf4_linear_forward_noalloc(const void *x, int64_t m, const nf4_weight *w,
                                      const void *lora_a, const void *lora_b, int32_t r,
                                      float lora_scale, void *y, void *stream);

/* Input gradient of the same linear ([MF] "Gradient Computation", the
 * activation-gradient equation):
 *   dX = dY . dequantize(W) + lora_scale * (dY . B^T) . A^T
 *   dy  device bf16 [m x N];  dx device bf16 [m x K] out.
 * Same operand, precision and workspace rules as nf4_linear_forward. */
nf4_status nf4_linear_backward_input(const void *dy, int64_t m, const nf4_weight *w,
                                     const void *lora_a, const void *lora_b, int32_t r,
                                     float lora_scale, void *dx, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* The kernel family that nf4_linear_forward (backward == 0) or
 * nf4_linear_backward_input (backward != 0) runs for m activation rows, a
 * weight [n_out x k_in] and adapter rank r. A host-only query; it launches
 * nothing and needs no device.
 *   NF4_LINEAR_DECODE    forward only, r == 0, 1 <= m <= 16, k_in % 256 == 0
 *                        and k_in <= 32768: the decode kernels, which stream
 *                        the weight once
 *   NF4_LINEAR_MFMA      n_out % 64 == 0 and r % 8 == 0: the bf16 matrix-core
 *                        GEMM, its adapter product on the matrix cores too
 *   NF4_LINEAR_PORTABLE  every other shape: a tiled fp32 kernel without the
 *                        matrix cores, one to two orders of magnitude slower
 *                        than the MFMA path at the same size (the same
 *                        results within the same tolerance)
 * Returns -1 for a shape the calls reject with NF4_ERR_SIZE (m < 0,
 * n_out < 1, k_in < 1 or not a multiple of 64, r outside 0..256). */
typedef enum { NF4_LINEAR_DECODE = 1, NF4_LINEAR_MFMA = 2, NF4_LINEAR_PORTABLE = 3 } nf4_linear_path;
int32_t nf4_linear_kernel_path(int64_t m, int64_t n_out, int64_t k_in, int32_t r, int32_t backward);

/* Bytes of device workspace that nf4_lora_backward needs: with rp = r rounded
 * up to 64 and mq = m rounded up to 64 plus 64, the bf16 products X.A and
 * dY.B^T (room for [mq x rp] each, rounded up to 256 bytes: they are stored
 * transposed with padded rows), then 8 fp32 partial sums of the larger of
 * 2 x [m x rp] and [k_in x r] + [r x n_out] (both products, or both gradients,
 * are split at once). No initialization is needed. Returns 0 for invalid
 * sizes. */
size_t nf4_lora_backward_workspace_size(int64_t m, int64_t k_in, int64_t n_out, int32_t r);

/* Gradients of the low-rank adapter of the same linear ([MF] "Gradient
 * Computation", the two adapter equations; A = L1 [k_in x r], B = L2 [r x n_out]):
 *   grad_a = lora_scale * X^T . (dY . B^T)      [k_in x r]
 *   grad_b = lora_scale * (X . A)^T . dY        [r x n_out]
 *   x        device bf16 [m x k_in] row-major (the forward's input)
 *   dy       device bf16 [m x n_out] (the gradient of the forward's output)
 *   lora_a   device bf16 [k_in x r];  lora_b  device bf16 [r x n_out]
 *   grad_a, grad_b  device out, row-major, fp32 or bf16 (grad_dtype); either may
 *            be NULL to skip it
 * bf16 operands; X.A and dY.B^T are rounded to bf16, the sums over the m
 * tokens accumulate in fp32. k_in % 64 == 0, n_out % 64 == 0, r % 8 == 0,
 * 8 <= r <= 256. m == 0 gives zero gradients. workspace: device, 256-byte
 * aligned, >= nf4_lora_backward_workspace_size(m, k_in, n_out, r) bytes; calls
 * that overlap in time must not share one. */
nf4_status nf4_lora_backward(const void *x, const void *dy, int64_t m, int64_t k_in, int64_t n_out,
                             const void *lora_a, const void *lora_b, int32_t r, float lora_scale,
                             void *grad_a, void *grad_b, int32_t grad_dtype, void *workspace,
                             size_t workspace_bytes, void *stream);

/* Bytes of device workspace nf4_merge_lora needs: the fp32 block scales of the
 * merged weight (n_out * k_in / 64 floats, rounded up to 256 bytes), used when
 * the merged weight is double-quantized and absmax_out is NULL. Returns 0 for
 * invalid sizes. */
size_t nf4_merge_lora_workspace_size(int64_t n_out, int64_t k_in);

/* Merges the low-rank adapter into the quantized base and re-quantizes
 * ([QP] "Step 4: Merging and Inference"; "QLoRA: quantising the part you are
 * not training" (addaly), "What it costs", item 3: merging into the quantized
 * base has to re-quantize). With W' = dequantize(w) in fp32:
 *   Wm[n][k] = fl32(W'[n][k] + fl32(lora_scale * d[n][k])),  d = (A . B)^T [N x K]
 * d is accumulated in fp32 on the matrix cores from the bf16 adapter (every
 * product exact, the order of the sum over the rank unspecified), then Wm is
 * quantized blockwise exactly as nf4_quantize does (codes_out, absmax_out),
 * and double-quantized as nf4_double_quantize does when absmax_q_out and
 * absmax_scale_out are given.
 *   w          the base: default format (B1 = 64; B2 = 256 if double-quantized)
 *   lora_a     device bf16 [k_in x r], 16-byte aligned; lora_b device bf16 [r x n_out]
 *   codes_out  device out, n_out * k_in / 2 bytes, 16-byte aligned
 *   absmax_out device out or NULL, one float per 64 weights
 *   absmax_q_out, absmax_scale_out  device out or both NULL (then absmax_out is required)
 *   workspace  >= nf4_merge_lora_workspace_size bytes, 256-byte aligned, when
 *              double quantization is requested without absmax_out; else may be NULL
 * The outputs may be the base's own buffers (in-place merge). k_in % 64 == 0,
 * r % 8 == 0, 8 <= r <= 256. */
nf4_status nf4_merge_lora(const nf4_weight *w, const void *lora_a, const void *lora_b, int32_t r,
                          float lora_scale, uint8_t *codes_out, float *absmax_out,
                          uint8_t *absmax_q_out, float *absmax_scale_out, void *workspace,
                          size_t workspace_bytes, void *stream);

/* ---- Storage-format variants ----
 * The entry points above fix B1 = 64, B2 = 256 and the E4M3FN code. [MF]
 * "Block-Wise Quantization Mechanics" gives 64 as the typical block size, and
 * [MF] "Double Quantization (DQ)" names neither the 8-bit float format nor
 * how its prose's asymmetric bias / mean subtraction is applied; the calls
 * below take these as parameters.
 *
 * Format of the second-level (8-bit) code of c1:
 *   NF4_DQ_E4M3     OCP FP8 E4M3FN of fl32(x / c2), round to nearest even
 *   NF4_DQ_E5M2     OCP FP8 E5M2 of fl32(x / c2), round to nearest even
 *   NF4_DQ_LINEAR8  uniform integer code: absmax_scale holds the step
 *                   u = fl32(c2 / L), L = 255 (127 with the mean offset), and
 *                   the code is rint(fl32(x / u)) clamped to [-L, L]
 * where x = c1, or x = fl32(c1 - mu) with the mean offset, and c2 = max |x|
 * over the group. With the mean offset the codes are signed (FP8 sign bit, or
 * int8 two's complement for NF4_DQ_LINEAR8) and mu = fl32(S / fl32(nblocks))
 * is one fp32 per tensor, S the pairwise fp32 sum of all c1 (the values
 * padded with zeros to a power-of-two count, adjacent pairs added level by
 * level). The reconstructed scale is
 *   scale(b) = fl32(decode(absmax_q[b]) * absmax_scale[b / B2])     (+ mu: one more fl32 add)
 * and the weight fl32(q[code] * scale(i / B1)) as before. */
typedef enum { NF4_DQ_E4M3 = 0, NF4_DQ_E5M2 = 1, NF4_DQ_LINEAR8 = 2 } nf4_dq_format;

/* The 16 levels of the 4-bit code ([MF] "Empirical Performance and
 * Architectural Guidelines" compares NF4 with FP4 and Int4; [QP] "1. 4-bit
 * NormalFloat (NF4)" compares it with a naive uniform 4-bit quantizer):
 *   NF4_CODEBOOK_NF4   the printed NF4 list (nf4_codebook())
 *   NF4_CODEBOOK_FP4   OCP FP4 (E2M1) in its own encoding, each value
 *                      fl32(v / 6): code = 8 * sign + the index of the
 *                      magnitude in 0, 0.5, 1, 1.5, 2, 3, 4, 6 (OCP
 *                      Microscaling Formats specification, the E2M1 table);
 *                      +0 is code 0 and -0 code 8 (equal to code 0, so never
 *                      chosen)
 *   NF4_CODEBOOK_INT4  fl32((2k - 15) / 15), k = 0..15: evenly spaced, no zero
 * A code is the index of the nearest level (lower index on a tie), and a
 * block with c1 == 0 gets the code of the level nearest 0. */
typedef enum { NF4_CODEBOOK_NF4 = 0, NF4_CODEBOOK_FP4 = 1, NF4_CODEBOOK_INT4 = 2 } nf4_codebook_id;

typedef struct {
    int32_t blocksize;      /* B1: a power of two in [16, 4096] */
    int32_t dq_blocksize;   /* B2: a power of two in [1, 4096] */
    int32_t dq_format;      /* an nf4_dq_format */
    int32_t dq_mean_offset; /* 0, or 1 for the tensor-wide mean offset */
    int32_t codebook;       /* an nf4_codebook_id */
} nf4_format;

/* The 16 levels of a codebook (static host array), NULL for an unknown id. */
const float *nf4_codebook_levels(int32_t codebook);

/* Bytes of the packed storage of an n-element tensor in format f: codes plus
 * either fp32 absmax (double_quant == 0) or the 8-bit codes, the fp32 group
 * values and, with the mean offset, one fp32 offset. Returns -1 for invalid
 * arguments. */
int64_t nf4_storage_bytes_ex(int64_t n, const nf4_format *f, int32_t double_quant);

/* Device workspace bytes of nf4_quantize_ex for an n-element tensor: fp32
 * block scales when the call runs in two passes (B1 != 64, B2 != 256 or the
 * mean offset, with double quantization) plus, with the mean offset, the
 * partial sums of mu. 0 when none is needed; (size_t)-1 for invalid args. */
size_t nf4_quantize_ex_workspace_size(int64_t n, const nf4_format *f);

/* Blockwise NF4 quantization with block size f->blocksize and, when absmax_q
 * and absmax_scale are given, double quantization in f's format (see above).
 *   w, codes, absmax, absmax_q, absmax_scale  as nf4_quantize, with B1, B2 of f
 *   absmax_offset  device out, one float (mu); required iff f->dq_mean_offset
 *                  and double quantization is on, else ignored
 *   workspace      device, 256-byte aligned, >= nf4_quantize_ex_workspace_size
 *                  bytes (may be NULL when that is 0)
 * The 4-bit codes index f->codebook's levels.
 * f = {64, 256, NF4_DQ_E4M3, 0, NF4_CODEBOOK_NF4} computes exactly what
 * nf4_quantize does. */
nf4_status nf4_quantize_ex(const void *w, int32_t w_dtype, int64_t n, const nf4_format *f,
                           uint8_t *codes, float *absmax, uint8_t *absmax_q, float *absmax_scale,
                           float *absmax_offset, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Device workspace bytes of nf4_double_quantize_ex (the partial sums of mu;
 * 0 without the mean offset); (size_t)-1 for invalid args. */
size_t nf4_double_quantize_ex_workspace_size(int64_t nblocks, const nf4_format *f);

/* Double quantization of nblocks existing fp32 block scales in f's format
 * (f->blocksize is not used). absmax_offset: device out, one float, required
 * iff f->dq_mean_offset. As in nf4_double_quantize, the values must be
 * finite, and the FP8 formats encode a negative value with the sign bit;
 * the unsigned linear code (NF4_DQ_LINEAR8 without the mean offset) takes
 * non-negative values only (a negative one is outside the contract). */
nf4_status nf4_double_quantize_ex(const float *absmax, int64_t nblocks, const nf4_format *f,
                                  uint8_t *absmax_q, float *absmax_scale, float *absmax_offset,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Dequantization of a tensor stored in format f (levels of f->codebook):
 * scale(b) as above, absmax
 * (fp32, no double quantization) when absmax_q == NULL. absmax_offset: device,
 * one float, required iff f->dq_mean_offset and absmax_q != NULL. */
nf4_status nf4_dequantize_ex(const uint8_t *codes, int64_t n, const nf4_format *f,
                             const float *absmax, const uint8_t *absmax_q,
                             const float *absmax_scale, const float *absmax_offset, void *out,
                             int32_t out_dtype, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* NF4_H */
