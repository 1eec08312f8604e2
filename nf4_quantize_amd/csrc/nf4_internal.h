// nf4_internal.h - internal declarations of the gfx950 NF4 library (not part
// of the C ABI). Shared by the library's own sources only.
//
// Sources (web pages), cited by title and section:
//   [MF] "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization,
//        Double Quantization, and Paged Optimizers" (llms.blog)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4.h"

namespace nf4 {

constexpr int kBlock = 64;                  // B1, [MF] "Block-Wise Quantization Mechanics"
constexpr int kDqBlock = 256;               // B2, [MF] "Double Quantization (DQ)"
constexpr int kGroup = kBlock * kDqBlock;   // 16384 weights share one c2

// The 16 NF4 levels, [MF] "4-Bit NormalFloat (NF4)" (the printed list).
extern const float kLevels[16];

// Nearest-level lookup. A normalised value v in [-1, 1] is bucketed by
//   offset(v) = bits(fl(v * 128 + (128 + 2^23))) & 0x1F8:
// the fma result lies in [2^23, 2^24), where the float's ulp is 1, so its
// low mantissa bits hold i = round(128 v + 128) and the mask keeps 8 * (i / 8),
// the byte offset of an 8-byte table entry (bucket k = i / 8, about 1/16 wide).
// No bucket holds more than one switch point of the code function, so
//   code(v) = hi[k] - (v < thr[k]),
// where hi[k] is the code at the top of the bucket and thr = -2.0 in a bucket
// without a switch point (hi - 1 >= 0 wherever v < thr can hold, so a word of
// packed hi nibbles minus the packed comparison bits never borrows across
// nibbles). For |v| <= 1 + 2^-20
// the bucket is 0..32; any input, NaN included, gives an offset below 512,
// so the table has 64 entries. Built on the host from the codebook by
// nf4::code_lut() (which buckets with this same fp32 formula) and passed to
// kernels by value.
constexpr int kLutEntries = 64;
constexpr int kLutUsed = 33;
struct LutEntry {
    float thr;
    int32_t hi;
};
struct CodeLut {
    LutEntry e[kLutEntries];
    // 1 for codebooks whose switch points are ratios of small integers (FP4,
    // Int4): bf16 quotients land on or next to them often, so the bf16 path
    // refines the quotient to fl32(w / c1) instead of falling back to the
    // division near a switch point.
    int32_t refine;
    // 1 for a sign-magnitude codebook (FP4 in the OCP E2M1 encoding: code
    // 8 + m is the negative of magnitude code m, 0 and 8 are +0 and -0). The
    // table then encodes the code of |v|, which is monotone; a negative v
    // with a non-zero magnitude code m gets 8 + m, and every v nearest zero
    // gets +0, the lower index of the +0 / -0 tie.
    int32_t signmag;
};
__host__ __device__ __forceinline__ uint32_t lut_offset_bits(float fma_result) {
    return __builtin_bit_cast(uint32_t, fma_result) & 0x1F8u;
}
// Returns the table of the NF4 levels, or of codebook `cb` (nf4_codebook_id),
// built once (thread-safe); nullptr if the codebook failed the construction
// checks or is unknown.
const CodeLut *code_lut();
const CodeLut *code_lut_for(int cb);
// The 16 levels of codebook `cb`, or nullptr.
const float *levels_for(int cb);

// |q - n| bound used by the quantize kernels: with r within 1 ulp of 1/c1,
// q = fl(w * r) and n = fl(w / c1) differ by less than 2.4e-7 for |w| <= c1;
// a q closer than kNearTol (9.5e-7) to a switch point is re-done with the
// correctly rounded division.
constexpr float kNearTol = 0x1p-20f;

// ---- internal launchers (host side; each validates nothing) ----
hipError_t launch_quantize(const void *w, nf4_dtype dt, int64_t n, uint8_t *codes, float *absmax,
                           uint8_t *absmax_q, float *absmax_scale, hipStream_t s);
hipError_t launch_double_quantize(const float *absmax, int64_t nblocks, uint8_t *absmax_q,
                                  float *absmax_scale, hipStream_t s);
hipError_t launch_dequantize(const uint8_t *codes, int64_t n, const float *absmax,
                             const uint8_t *absmax_q, const float *absmax_scale, void *out,
                             nf4_dtype dt, hipStream_t s);
// Storage-format variants: block size B1, DQ block B2, the 8-bit code format
// of double quantization and the tensor-wide mean offset (nf4_format).
// Batched storage path (B1 = 64, B2 = 256, E4M3): the entries' full groups
// in launches of up to 32 entries, their partial groups in one more.
hipError_t launch_quantize_batched(const nf4_batch_entry *e, int32_t count, nf4_dtype dt,
                                   hipStream_t s);
hipError_t launch_dequantize_batched(const nf4_batch_entry *e, int32_t count, nf4_dtype dt,
                                     hipStream_t s);
hipError_t launch_quantize_ex(const void *w, nf4_dtype dt, int64_t n, const nf4_format &f,
                              uint8_t *codes, float *absmax, uint8_t *absmax_q,
                              float *absmax_scale, float *absmax_offset, void *workspace,
                              hipStream_t s);
hipError_t launch_double_quantize_ex(const float *absmax, int64_t nblocks, const nf4_format &f,
                                     uint8_t *absmax_q, float *absmax_scale,
                                     float *absmax_offset, void *workspace, hipStream_t s,
                                     const float *parts = nullptr, int64_t nparts = 0);
hipError_t launch_dequantize_ex(const uint8_t *codes, int64_t n, const nf4_format &f,
                                const float *absmax, const uint8_t *absmax_q,
                                const float *absmax_scale, const float *absmax_offset, void *out,
                                nf4_dtype dt, hipStream_t s);
// Workspace of the variants: fp32 block scales (when they are not an output
// of a two-pass quantization) and the partial sums of the mean offset.
size_t quantize_ex_workspace(int64_t n, const nf4_format &f);
size_t double_quantize_ex_workspace(int64_t nblocks, const nf4_format &f);
// Merging the adapter into the quantized base (W [N x K] default format).
size_t merge_workspace(int64_t n_out, int64_t k_in);
hipError_t launch_merge(const nf4_weight &w, const uint16_t *a, const uint16_t *b, int32_t r,
                        float s_lora, uint8_t *codes_out, float *absmax_out, uint8_t *absmax_q_out,
                        float *absmax_scale_out, void *workspace, hipStream_t s);
// The kernel family (nf4_linear_path) a linear call of this shape runs;
// the launchers below dispatch by it.
nf4_linear_path linear_path(int64_t m, int64_t n_out, int64_t k_in, int32_t r, bool backward);
hipError_t launch_linear_forward(const uint16_t *x, int64_t m, const nf4_weight &w,
                                 const uint16_t *a, const uint16_t *b, int32_t r, float s_lora,
                                 uint16_t *y, void *workspace, hipStream_t s);
hipError_t launch_linear_backward_input(const uint16_t *dy, int64_t m, const nf4_weight &w,
                                        const uint16_t *a, const uint16_t *b, int32_t r,
                                        float s_lora, uint16_t *dx, void *workspace,
                                        hipStream_t s);

// ---- device helpers ----

// Native 16-byte vectors (usable with the nontemporal load/store builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 bits -> fp32 (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even; gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// OCP FP8 E4M3FN decode of a non-negative code (bias 7, 3 mantissa bits;
// exponent field 0 is subnormal m * 2^-9).
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (c & 0x80u) ? -v : v;
}

// OCP FP8 E4M3FN encode of r in [0, 1], round to nearest, ties to even.
// Below 2^-6 the format is uniform with step 2^-9, so the code is the
// rounded multiple of the step; above, the 23-bit mantissa is cut to 3 bits
// and a round-up carries into the exponent because codes are monotone.
__device__ __forceinline__ uint32_t e4m3_encode_unit(float r) {
    uint32_t u = __float_as_uint(r);
    if (u < 0x3C800000u) return (uint32_t)__builtin_rintf(r * 512.0f);
    int e = (int)(u >> 23) - 127;
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
    uint32_t up = (rest > 0x80000u) | ((rest == 0x80000u) & (keep & 1u));
    return (uint32_t)((e + 7) << 3) + keep + up;
}

// OCP FP8 E5M2 encode of r in [0, 1], round to nearest, ties to even (5
// exponent bits, bias 15, 2 mantissa bits; below 2^-14 uniform with step 2^-16).
__device__ __forceinline__ uint32_t e5m2_encode_unit(float r) {
    uint32_t u = __float_as_uint(r);
    if (u < 0x38800000u) return (uint32_t)__builtin_rintf(r * 65536.0f);
    int e = (int)(u >> 23) - 127;
    uint32_t mant = u & 0x7FFFFFu;
    uint32_t keep = mant >> 21, rest = mant & 0x1FFFFFu;
    uint32_t up = (rest > 0x100000u) | ((rest == 0x100000u) & (keep & 1u));
    return (uint32_t)((e + 15) << 2) + keep + up;
}

// The 8-bit code of double quantization (nf4_dq_format), kS = signed codes
// (mean offset on). x is c1 (or c1 - mu), sc the stored group value: c2 for
// the float formats, the step c2 / L for the linear code (L = 255, 127 signed).
enum : int { kFmtE4M3 = NF4_DQ_E4M3, kFmtE5M2 = NF4_DQ_E5M2, kFmtLin8 = NF4_DQ_LINEAR8 };
template <bool kS> constexpr float lin_levels() { return kS ? 127.0f : 255.0f; }

template <int F, bool kS>
__device__ __forceinline__ uint32_t dq_encode(float x, float sc) {
    if constexpr (F == kFmtLin8) {
        if (sc == 0.0f) return 0u;
        const float l = lin_levels<kS>();
        const float t = fminf(fmaxf(__builtin_rintf(x / sc), -l), l);
        return (uint32_t)(int)t & 0xFFu;
    } else {
        // the FP8 formats carry a sign: a negative ratio (a signed scale, or
        // c1 - mu with the mean offset) is its magnitude's code plus bit 7
        const float r = (sc == 0.0f) ? 0.0f : x / sc;
        const uint32_t sign = signbit(r) ? 0x80u : 0u;
        const float a = fabsf(r);
        return sign | (F == kFmtE5M2 ? e5m2_encode_unit(a) : e4m3_encode_unit(a));
    }
}

// Decode of the code in byte J of v (gfx950's fp8 / bf8 converts decode OCP
// E4M3FN / E5M2, sign included).
template <int F, bool kS, int J = 0>
__device__ __forceinline__ float dq_decode(uint32_t v) {
    if constexpr (F == kFmtE4M3) return __builtin_amdgcn_cvt_f32_fp8((int)v, J);
    else if constexpr (F == kFmtE5M2) return __builtin_amdgcn_cvt_f32_bf8((int)v, J);
    else if constexpr (kS) return (float)(int)(int8_t)(uint8_t)(v >> (8 * J));
    else return (float)((v >> (8 * J)) & 0xFFu);
}

// Reconstructed first-level scale c1' of one block.
__device__ __forceinline__ float block_scale(int64_t b, const float *absmax, const uint8_t *q,
                                             const float *scale) {
    if (q == nullptr) return absmax[b];
    return e4m3_decode(q[b]) * scale[b / kDqBlock];
}

}  // namespace nf4
