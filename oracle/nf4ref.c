/*
 * nf4ref.c - CPU oracle for blockwise NF4 quantization, double quantization,
 * dequantization and the QLoRA linear (forward and input gradient).
 *
 * TEST INFRASTRUCTURE ONLY: plain, slow, single-threaded C11, written step by
 * step from the defining equations. It is built with -O2 -ffp-contract=off and
 * no fast-math, so every float operation below is one IEEE-754 binary32
 * operation rounded to nearest even (x86-64 SSE, FLT_EVAL_METHOD == 0).
 * It shares no code with the GPU library. Source keys are listed in nf4ref.h.
 *
 * Readings where the pages are silent (each is also listed with its reason in
 * the design notes of the repository):
 *   - division w/c1 and c1/c2 are correctly rounded fp32 divisions;
 *   - the argmin is taken over fp32 distances |fl32(n - q_i)|, lowest index on ties;
 *   - a block with c1 == 0 gets code 7 (the exact zero level) everywhere;
 *   - the double-quantization 8-bit format is OCP FP8 E4M3FN, round to nearest
 *     even; c2 == 0 gives code 0 for every block of the group;
 *   - the reconstructed scale is fl32(decode(code8) * c2), then the weight is
 *     fl32(q[code] * scale); bf16 output rounds that fp32 value to nearest even;
 *   - non-finite inputs are outside the contract and rejected (-2).
 */
#include "nf4ref.h"

#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

_Static_assert(FLT_EVAL_METHOD == 0, "float expressions must evaluate in binary32");

/* [MF] "4-Bit NormalFloat (NF4)": the printed list q_0 .. q_15. Each printed
 * decimal is an exact binary32 value. */
static const float NF4_Q[16] = {
    -1.0f,
    -0.6961928009986877f,
    -0.5250730514526367f,
    -0.39491748809814453f,
    -0.28444138169288635f,
    -0.18477343022823334f,
    -0.09105003625154495f,
    0.0f,
    0.07958029955625534f,
    0.16093020141124725f,
    0.24611230194568634f,
    0.33791524171829224f,
    0.44070982933044434f,
    0.5626170039176941f,
    0.7229568362236023f,
    1.0f,
};

void nf4ref_codebook(float q[16]) {
    for (int i = 0; i < 16; ++i) q[i] = NF4_Q[i];
}

/* ---- codebook construction check ([MF] "4-Bit NormalFloat (NF4)") ---- */

/* Lower-tail probability P(Z <= x) of the standard normal. */
static double std_normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

double nf4ref_normal_quantile(double p) {
    if (!(p > 0.0 && p < 1.0)) return NAN;
    /* Bisect on the smaller tail (1 - p is exact for p >= 1/2), then use the
     * symmetry quantile(p) = -quantile(1 - p). */
    double tail = p < 0.5 ? p : 1.0 - p;
    double lo = -40.0, hi = 0.0;
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        if (std_normal_cdf(mid) < tail)
            lo = mid;
        else
            hi = mid;
    }
    double x = 0.5 * (lo + hi);
    return p < 0.5 ? x : -x;
}

int nf4ref_construct_codebook(double delta, double out[16]) {
    if (!out || !(delta > 0.5 && delta < 1.0)) return -1;
    /* Positive half: 8 levels at probabilities delta - i*(delta-1/2)/8, i=0..7
     * (the 9th point of that grid is 1/2, whose quantile is the zero level).
     * Negative half: 7 levels at delta - j*(delta-1/2)/7, j=0..6, mirrored. */
    double top = nf4ref_normal_quantile(delta);
    for (int i = 0; i < 8; ++i) {
        double p = delta - (double)i * (delta - 0.5) / 8.0;
        out[15 - i] = nf4ref_normal_quantile(p) / top;
    }
    out[7] = 0.0;
    for (int j = 0; j < 7; ++j) {
        double p = delta - (double)j * (delta - 0.5) / 7.0;
        out[j] = -nf4ref_normal_quantile(p) / top;
    }
    return 0;
}

double nf4ref_solve_delta(double level14) {
    double lo = 0.9, hi = 0.9999, v[16];
    /* Level 14 of the construction decreases as delta grows on this interval:
     * the normaliser quantile(delta) grows faster than quantile of the next
     * probability down. */
    for (int it = 0; it < 200; ++it) {
        double mid = 0.5 * (lo + hi);
        if (mid == lo || mid == hi) break;
        nf4ref_construct_codebook(mid, v);
        if (v[14] > level14)
            lo = mid;
        else
            hi = mid;
    }
    return 0.5 * (lo + hi);
}

/* ---- nearest level ([MF] "Block-Wise Quantization Mechanics", argmin) ---- */

int nf4ref_nearest_code(float n) {
    int best = 0;
    float best_d = fabsf(n - NF4_Q[0]);
    for (int i = 1; i < 16; ++i) {
        float d = fabsf(n - NF4_Q[i]);
        if (d < best_d) { /* strict: on equal distance the lower index stays */
            best_d = d;
            best = i;
        }
    }
    return best;
}

int nf4ref_nearest_code_array(const float *n, int64_t count, uint8_t *out) {
    if (count < 0 || (count > 0 && (!n || !out))) return -1;
    for (int64_t i = 0; i < count; ++i) out[i] = (uint8_t)nf4ref_nearest_code(n[i]);
    return 0;
}

/* ---- bf16 ---- */

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}
static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

float nf4ref_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

uint16_t nf4ref_f32_to_bf16(float f) {
    /* bf16 keeps the upper 16 bits of binary32. The two candidates are the
     * truncation and the next value up in magnitude; pick the nearer, and on
     * an exact halfway point the one whose last kept bit is 0. */
    uint32_t u = f32_bits(f);
    uint32_t down = u & 0xFFFF0000u;
    uint32_t rest = u & 0x0000FFFFu;
    uint32_t up = down + 0x00010000u;
    uint32_t pick;
    if (rest > 0x8000u)
        pick = up;
    else if (rest < 0x8000u)
        pick = down;
    else
        pick = ((down >> 16) & 1u) ? up : down;
    return (uint16_t)(pick >> 16);
}

int nf4ref_f32_to_bf16_array(const float *x, int64_t n, uint16_t *out) {
    if (n < 0 || (n > 0 && (!x || !out))) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = nf4ref_f32_to_bf16(x[i]);
    return 0;
}

/* ---- blockwise quantization ([MF] "Block-Wise Quantization Mechanics") ---- */

static float load_elem(const void *w, int dtype, int64_t i) {
    if (dtype == NF4REF_F32) return ((const float *)w)[i];
    return nf4ref_bf16_to_f32(((const uint16_t *)w)[i]);
}

static int pow2_in(int64_t v, int64_t lo, int64_t hi) {
    return v >= lo && v <= hi && (v & (v - 1)) == 0;
}

int nf4ref_quantize_bs(const void *w, int dtype, int64_t n, int32_t blocksize, uint8_t *codes,
                       float *absmax) {
    if (n < 0 || !pow2_in(blocksize, 16, 4096)) return -1;
    if (n == 0) return 0;
    if (!w || !codes || !absmax) return -1;
    if (dtype != NF4REF_F32 && dtype != NF4REF_BF16) return -1;
    int64_t nblocks = (n + blocksize - 1) / blocksize;
    memset(codes, 0, (size_t)((n + 1) / 2));
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * blocksize;
        int64_t hi = lo + blocksize < n ? lo + blocksize : n;
        /* c1 = max |w| over the block. */
        float c1 = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float v = load_elem(w, dtype, i);
            if (!isfinite(v)) return -2;
            if (fabsf(v) > c1) c1 = fabsf(v);
        }
        absmax[b] = c1;
        for (int64_t i = lo; i < hi; ++i) {
            int code;
            if (c1 == 0.0f) {
                code = 7; /* the exact zero level */
            } else {
                float nrm = load_elem(w, dtype, i) / c1;
                code = nf4ref_nearest_code(nrm);
            }
            codes[i / 2] |= (uint8_t)(code << (4 * (int)(i & 1)));
        }
    }
    return 0;
}

int nf4ref_quantize(const void *w, int dtype, int64_t n, uint8_t *codes, float *absmax) {
    return nf4ref_quantize_bs(w, dtype, n, NF4REF_BLOCK, codes, absmax);
}

/* ---- OCP FP8 E4M3FN ---- */

uint8_t nf4ref_e4m3_encode(float r) {
    /* E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity,
     * largest finite 448. Round to nearest, ties to even mantissa. Codes of
     * non-negative values are monotone in value, so a mantissa that rounds up
     * to 8 carries into the exponent by plain addition. */
    uint8_t sign = 0;
    double v = (double)r;
    if (isnan(r)) return 0x7F;
    if (signbit(r)) { /* negative values and -0 keep the sign bit */
        sign = 0x80;
        v = -v;
    }
    if (v == 0.0) return sign;
    if (v >= 464.0) return (uint8_t)(sign | 0x7E); /* beyond max + half step: saturate */
    uint8_t code;
    if (v < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9, m = 0..7; m == 8 is code 0x08 = 2^-6 */
        code = (uint8_t)rint(v * 512.0);
    } else {
        int e2;
        double f = frexp(v, &e2); /* v = f * 2^e2, f in [0.5, 1) */
        int e = e2 - 1;           /* v = s * 2^e, s in [1, 2) */
        double s = 2.0 * f;
        int mant = (int)rint((s - 1.0) * 8.0);
        int c = ((e + 7) << 3) + mant;
        if (c > 0x7E) c = 0x7E;
        code = (uint8_t)c;
    }
    return (uint8_t)(sign | code);
}

float nf4ref_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1;
    int e = (c >> 3) & 15;
    int m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

int nf4ref_e4m3_encode_array(const float *r, int64_t n, uint8_t *out) {
    if (n < 0 || (n > 0 && (!r || !out))) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = nf4ref_e4m3_encode(r[i]);
    return 0;
}

/* ---- double quantization ([MF] "Double Quantization (DQ)") ---- */

int nf4ref_double_quantize(const float *absmax, int64_t nblocks, uint8_t *q, float *scale) {
    if (nblocks < 0) return -1;
    if (nblocks == 0) return 0;
    if (!absmax || !q || !scale) return -1;
    int64_t ngroups = (nblocks + NF4REF_DQ_BLOCK - 1) / NF4REF_DQ_BLOCK;
    for (int64_t g = 0; g < ngroups; ++g) {
        int64_t lo = g * NF4REF_DQ_BLOCK;
        int64_t hi = lo + NF4REF_DQ_BLOCK < nblocks ? lo + NF4REF_DQ_BLOCK : nblocks;
        float c2 = 0.0f;
        for (int64_t b = lo; b < hi; ++b) {
            if (!isfinite(absmax[b])) return -2;
            if (fabsf(absmax[b]) > c2) c2 = fabsf(absmax[b]);
        }
        scale[g] = c2;
        for (int64_t b = lo; b < hi; ++b) {
            float ratio = (c2 == 0.0f) ? 0.0f : absmax[b] / c2;
            q[b] = nf4ref_e4m3_encode(ratio);
        }
    }
    return 0;
}

/* ---- dequantization ([MF] "Block-Wise Quantization Mechanics", the
 *      reconstruction equation, and the dequantize(c1, c2, W) of
 *      "Forward Pass Computation") ---- */

float nf4ref_block_scale(int64_t b, const float *absmax, const uint8_t *q, const float *scale) {
    if (!q) return absmax[b];
    return nf4ref_e4m3_decode(q[b]) * scale[b / NF4REF_DQ_BLOCK];
}

int nf4ref_dequantize_range(const uint8_t *codes, int64_t n, int64_t start, int64_t count,
                            const float *absmax, const uint8_t *q, const float *scale, void *out,
                            int out_dtype) {
    if (n < 0 || start < 0 || count < 0 || start + count > n) return -1;
    if (count == 0) return 0;
    if (!codes || !out) return -1;
    if (!q && !absmax) return -1;
    if (q && !scale) return -1;
    if (out_dtype != NF4REF_F32 && out_dtype != NF4REF_BF16) return -1;
    for (int64_t j = 0; j < count; ++j) {
        int64_t i = start + j;
        int code = (codes[i / 2] >> (4 * (int)(i & 1))) & 15;
        float c1 = nf4ref_block_scale(i / NF4REF_BLOCK, absmax, q, scale);
        float v = NF4_Q[code] * c1;
        if (out_dtype == NF4REF_F32)
            ((float *)out)[j] = v;
        else
            ((uint16_t *)out)[j] = nf4ref_f32_to_bf16(v);
    }
    return 0;
}

int nf4ref_dequantize(const uint8_t *codes, int64_t n, const float *absmax, const uint8_t *q,
                      const float *scale, void *out, int out_dtype) {
    return nf4ref_dequantize_range(codes, n, 0, n, absmax, q, scale, out, out_dtype);
}

/* ---- variants of double quantization (see nf4ref.h) ---- */

/* OCP FP8 E5M2: sign, 5 exponent bits (bias 15), 2 mantissa bits; exponent
 * field 31 holds infinities and NaNs, the largest finite value is 57344.
 * Exponent field 0 is subnormal, m * 2^-16. */
uint8_t nf4ref_e5m2_encode(float r) {
    uint8_t sign = 0;
    double v = (double)r;
    if (isnan(r)) return 0x7F;
    if (signbit(r)) { /* negative values and -0 keep the sign bit */
        sign = 0x80;
        v = -v;
    }
    if (v == 0.0) return sign;
    if (v >= 61440.0) return (uint8_t)(sign | 0x7B); /* beyond max + half step: saturate */
    int code;
    if (v < ldexp(1.0, -14)) {
        code = (int)rint(v * 65536.0); /* m = 4 is code 0x04 = 2^-14 */
    } else {
        int e2;
        double f = frexp(v, &e2);
        int e = e2 - 1;
        int mant = (int)rint((2.0 * f - 1.0) * 4.0);
        code = ((e + 15) << 2) + mant;
        if (code > 0x7B) code = 0x7B;
    }
    return (uint8_t)(sign | code);
}

float nf4ref_e5m2_decode(uint8_t c) {
    int s = (c >> 7) & 1;
    int e = (c >> 2) & 31;
    int m = c & 3;
    double v;
    if (e == 31) v = m ? NAN : INFINITY;
    else if (e == 0) v = ldexp((double)m, -16);
    else v = ldexp(1.0 + (double)m / 4.0, e - 15);
    return (float)(s ? -v : v);
}

int nf4ref_e5m2_encode_array(const float *r, int64_t n, uint8_t *out) {
    if (n < 0 || (n > 0 && (!r || !out))) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = nf4ref_e5m2_encode(r[i]);
    return 0;
}

static float pairwise_node(const float *x, int64_t n, int64_t lo, int64_t len) {
    if (lo >= n) return 0.0f;
    if (len == 1) return x[lo];
    return pairwise_node(x, n, lo, len / 2) + pairwise_node(x, n, lo + len / 2, len / 2);
}

float nf4ref_pairwise_sum(const float *x, int64_t n) {
    if (n <= 0) return 0.0f;
    int64_t p = 1;
    while (p < n) p *= 2;
    return pairwise_node(x, n, 0, p);
}

/* Levels of the linear code: 255 unsigned, 127 signed. */
static float linear_levels(int mean_offset) { return mean_offset ? 127.0f : 255.0f; }

/* The 8-bit code of value x in the group with stored value sc (c2, or the
 * step u of the linear code). */
static uint8_t dq_encode(float x, float sc, int fmt, int mean_offset) {
    if (fmt == NF4REF_DQ_LINEAR8) {
        float lv = linear_levels(mean_offset);
        if (sc == 0.0f) return 0;
        float t = rintf(x / sc); /* nearest integer, ties to even */
        if (t > lv) t = lv;
        if (t < -lv) t = -lv;
        return (uint8_t)(int8_t)(int)t; /* two's complement when signed */
    }
    float ratio = (sc == 0.0f) ? 0.0f : x / sc;
    return fmt == NF4REF_DQ_E5M2 ? nf4ref_e5m2_encode(ratio) : nf4ref_e4m3_encode(ratio);
}

static float dq_decode(uint8_t c, int fmt, int mean_offset) {
    if (fmt == NF4REF_DQ_LINEAR8) return mean_offset ? (float)(int8_t)c : (float)c;
    return fmt == NF4REF_DQ_E5M2 ? nf4ref_e5m2_decode(c) : nf4ref_e4m3_decode(c);
}

int nf4ref_double_quantize_ex(const float *absmax, int64_t nblocks, int32_t dq_blocksize,
                              int dq_format, int mean_offset, uint8_t *q, float *scale,
                              float *offset) {
    if (nblocks < 0 || !pow2_in(dq_blocksize, 1, 4096)) return -1;
    if (dq_format < NF4REF_DQ_E4M3 || dq_format > NF4REF_DQ_LINEAR8) return -1;
    if (mean_offset && !offset) return -1;
    if (nblocks == 0) {
        if (mean_offset) *offset = 0.0f;
        return 0;
    }
    if (!absmax || !q || !scale) return -1;
    for (int64_t b = 0; b < nblocks; ++b) {
        if (!isfinite(absmax[b])) return -2;
        /* the unsigned linear code holds 0..255 steps of a non-negative c1
         * (a block absmax); it has no code for a negative scale */
        if (dq_format == NF4REF_DQ_LINEAR8 && !mean_offset && absmax[b] < 0.0f) return -1;
    }
    float mu = 0.0f;
    if (mean_offset) {
        mu = nf4ref_pairwise_sum(absmax, nblocks) / (float)nblocks;
        if (!isfinite(mu)) return -2;
        *offset = mu;
    }
    int64_t ngroups = (nblocks + dq_blocksize - 1) / dq_blocksize;
    for (int64_t g = 0; g < ngroups; ++g) {
        int64_t lo = g * dq_blocksize;
        int64_t hi = lo + dq_blocksize < nblocks ? lo + dq_blocksize : nblocks;
        /* c2 = max |x| over the group, x = c1 (or c1 - mu) */
        float c2 = 0.0f;
        for (int64_t b = lo; b < hi; ++b) {
            float x = mean_offset ? absmax[b] - mu : absmax[b];
            if (fabsf(x) > c2) c2 = fabsf(x);
        }
        float sc = (dq_format == NF4REF_DQ_LINEAR8) ? c2 / linear_levels(mean_offset) : c2;
        scale[g] = sc;
        for (int64_t b = lo; b < hi; ++b) {
            float x = mean_offset ? absmax[b] - mu : absmax[b];
            q[b] = dq_encode(x, sc, dq_format, mean_offset);
        }
    }
    return 0;
}

float nf4ref_block_scale_ex(int64_t b, int32_t dq_blocksize, int dq_format, const float *absmax,
                            const uint8_t *q, const float *scale, const float *offset) {
    if (!q) return absmax[b];
    float v = dq_decode(q[b], dq_format, offset != NULL) * scale[b / dq_blocksize];
    if (offset) v = v + *offset;
    return v;
}

int nf4ref_dequantize_range_ex(const uint8_t *codes, int64_t n, int64_t start, int64_t count,
                               int32_t blocksize, int32_t dq_blocksize, int dq_format,
                               const float *absmax, const uint8_t *q, const float *scale,
                               const float *offset, void *out, int out_dtype) {
    if (n < 0 || start < 0 || count < 0 || start + count > n) return -1;
    if (!pow2_in(blocksize, 16, 4096) || !pow2_in(dq_blocksize, 1, 4096)) return -1;
    if (dq_format < NF4REF_DQ_E4M3 || dq_format > NF4REF_DQ_LINEAR8) return -1;
    if (count == 0) return 0;
    if (!codes || !out) return -1;
    if (!q && !absmax) return -1;
    if (q && !scale) return -1;
    if (out_dtype != NF4REF_F32 && out_dtype != NF4REF_BF16) return -1;
    for (int64_t j = 0; j < count; ++j) {
        int64_t i = start + j;
        int code = (codes[i / 2] >> (4 * (int)(i & 1))) & 15;
        float c1 = nf4ref_block_scale_ex(i / blocksize, dq_blocksize, dq_format, absmax, q, scale,
                                         offset);
        float v = NF4_Q[code] * c1;
        if (out_dtype == NF4REF_F32)
            ((float *)out)[j] = v;
        else
            ((uint16_t *)out)[j] = nf4ref_f32_to_bf16(v);
    }
    return 0;
}

/* ---- merging the adapter into the quantized base (see nf4ref.h) ---- */

int nf4ref_merged_weight(const uint8_t *codes, const float *absmax, const uint8_t *q,
                         const float *scale, int64_t N, int64_t K, const uint16_t *A,
                         const uint16_t *B, int32_t r, float s, const int64_t *rows,
                         int64_t nrows, float *wm) {
    if (N <= 0 || K <= 0 || r < 0 || (r > 0 && (!A || !B)) || !codes || !wm) return -1;
    if (!q && !absmax) return -1;
    if (q && !scale) return -1;
    if (!rows) nrows = N;
    if (nrows < 0) return -1;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t n = rows ? rows[i] : i;
        if (n < 0 || n >= N) return -1;
        /* the dequantized row of the base */
        if (nf4ref_dequantize_range(codes, N * K, n * K, K, absmax, q, scale, wm + i * K,
                                    NF4REF_F32) != 0)
            return -1;
        for (int64_t k = 0; k < K; ++k) {
            double d = 0.0;
            for (int32_t j = 0; j < r; ++j)
                d += (double)nf4ref_bf16_to_f32(A[k * r + j]) *
                     (double)nf4ref_bf16_to_f32(B[(int64_t)j * N + n]);
            float d32 = (float)d;
            float delta = s * d32;
            wm[i * K + k] = wm[i * K + k] + delta;
        }
    }
    return 0;
}

/* ---- codebook swaps (see nf4ref.h) ---- */

int nf4ref_codebook_levels(int codebook, float q[16]) {
    if (!q) return -1;
    if (codebook == NF4REF_CB_NF4) {
        for (int i = 0; i < 16; ++i) q[i] = NF4_Q[i];
    } else if (codebook == NF4REF_CB_FP4) {
        /* OCP E2M1 encoding: bit 3 is the sign, bits 2..1 the exponent (bias
         * 1), bit 0 the mantissa; exponent 0 is subnormal (0 or 0.5). The
         * code's value divided by 6 puts the largest magnitude at 1. */
        for (int c = 0; c < 16; ++c) {
            const int e = (c >> 1) & 3, m = c & 1;
            const float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, e - 1);
            const float v = mag / 6.0f;
            q[c] = (c & 8) ? -v : v;  /* code 8 is -0 */
        }
    } else if (codebook == NF4REF_CB_INT4) {
        for (int k = 0; k < 16; ++k) q[k] = (float)(2 * k - 15) / 15.0f;
    } else {
        return -1;
    }
    return 0;
}

static int nearest_in(const float q[16], float n) {
    int best = 0;
    float best_d = fabsf(n - q[0]);
    for (int i = 1; i < 16; ++i) {
        float d = fabsf(n - q[i]);
        if (d < best_d) {
            best_d = d;
            best = i;
        }
    }
    return best;
}

int nf4ref_quantize_cb(const void *w, int dtype, int64_t n, int32_t blocksize, int codebook,
                       uint8_t *codes, float *absmax) {
    float q[16];
    if (nf4ref_codebook_levels(codebook, q) != 0) return -1;
    if (n < 0 || !pow2_in(blocksize, 16, 4096)) return -1;
    if (n == 0) return 0;
    if (!w || !codes || !absmax) return -1;
    if (dtype != NF4REF_F32 && dtype != NF4REF_BF16) return -1;
    const int zero_code = nearest_in(q, 0.0f);
    int64_t nblocks = (n + blocksize - 1) / blocksize;
    memset(codes, 0, (size_t)((n + 1) / 2));
    for (int64_t b = 0; b < nblocks; ++b) {
        int64_t lo = b * blocksize;
        int64_t hi = lo + blocksize < n ? lo + blocksize : n;
        float c1 = 0.0f;
        for (int64_t i = lo; i < hi; ++i) {
            float v = load_elem(w, dtype, i);
            if (!isfinite(v)) return -2;
            if (fabsf(v) > c1) c1 = fabsf(v);
        }
        absmax[b] = c1;
        for (int64_t i = lo; i < hi; ++i) {
            int code = (c1 == 0.0f) ? zero_code : nearest_in(q, load_elem(w, dtype, i) / c1);
            codes[i / 2] |= (uint8_t)(code << (4 * (int)(i & 1)));
        }
    }
    return 0;
}

int nf4ref_dequantize_range_cb(const uint8_t *codes, int64_t n, int64_t start, int64_t count,
                               int32_t blocksize, int32_t dq_blocksize, int dq_format, int codebook,
                               const float *absmax, const uint8_t *q, const float *scale,
                               const float *offset, void *out, int out_dtype) {
    float lv[16];
    if (nf4ref_codebook_levels(codebook, lv) != 0) return -1;
    if (n < 0 || start < 0 || count < 0 || start + count > n) return -1;
    if (!pow2_in(blocksize, 16, 4096) || !pow2_in(dq_blocksize, 1, 4096)) return -1;
    if (dq_format < NF4REF_DQ_E4M3 || dq_format > NF4REF_DQ_LINEAR8) return -1;
    if (count == 0) return 0;
    if (!codes || !out) return -1;
    if (!q && !absmax) return -1;
    if (q && !scale) return -1;
    if (out_dtype != NF4REF_F32 && out_dtype != NF4REF_BF16) return -1;
    for (int64_t j = 0; j < count; ++j) {
        int64_t i = start + j;
        int code = (codes[i / 2] >> (4 * (int)(i & 1))) & 15;
        float c1 = nf4ref_block_scale_ex(i / blocksize, dq_blocksize, dq_format, absmax, q, scale,
                                         offset);
        float v = lv[code] * c1;
        if (out_dtype == NF4REF_F32)
            ((float *)out)[j] = v;
        else
            ((uint16_t *)out)[j] = nf4ref_f32_to_bf16(v);
    }
    return 0;
}

/* ---- storage footprint ([L15] "Double quantisation" per-parameter tables) ---- */

int64_t nf4ref_storage_bytes(int64_t n, int dq) {
    if (n < 0) return -1;
    int64_t nblocks = (n + NF4REF_BLOCK - 1) / NF4REF_BLOCK;
    int64_t ngroups = (nblocks + NF4REF_DQ_BLOCK - 1) / NF4REF_DQ_BLOCK;
    int64_t code_bytes = (n + 1) / 2;
    if (!dq) return code_bytes + 4 * nblocks;
    return code_bytes + nblocks + 4 * ngroups;
}

/* ---- QLoRA linear ([MF] "Forward Pass Computation", "Gradient Computation") ---- */

int nf4ref_linear_forward(const uint16_t *x, int64_t m, int64_t K, int64_t N, const float *wdeq,
                          const uint16_t *A, const uint16_t *B, int32_t r, double s,
                          const int64_t *rows, int64_t nrows, const int64_t *cols, int64_t ncols,
                          double *out) {
    if (!x || !wdeq || !out || m < 0 || K < 0 || N < 0 || r < 0) return -1;
    int lora = (A != NULL && r > 0);
    if (lora && !B) return -1;
    if (!rows) nrows = m;
    if (!cols) ncols = N;
    double t[4096];
    if (r > 4096) return -1;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        if (row < 0 || row >= m) return -1;
        const uint16_t *xr = x + row * K;
        /* adapter down-projection of this row: t = x_row . A (r values) */
        if (lora) {
            for (int32_t c = 0; c < r; ++c) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += (double)nf4ref_bf16_to_f32(xr[k]) *
                           (double)nf4ref_bf16_to_f32(A[k * r + c]);
                t[c] = acc;
            }
        }
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t col = cols ? cols[j] : j;
            if (col < 0 || col >= N) return -1;
            const float *wr = wdeq + col * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)nf4ref_bf16_to_f32(xr[k]) * (double)wr[k];
            if (lora) {
                double side = 0.0;
                for (int32_t c = 0; c < r; ++c)
                    side += t[c] * (double)nf4ref_bf16_to_f32(B[(int64_t)c * N + col]);
                acc += s * side;
            }
            out[i * ncols + j] = acc;
        }
    }
    return 0;
}

int nf4ref_linear_backward_input(const uint16_t *dy, int64_t m, int64_t K, int64_t N,
                                 const float *wdeq, const uint16_t *A, const uint16_t *B,
                                 int32_t r, double s, const int64_t *rows, int64_t nrows,
                                 const int64_t *cols, int64_t ncols, double *out) {
    if (!dy || !wdeq || !out || m < 0 || K < 0 || N < 0 || r < 0) return -1;
    int lora = (A != NULL && r > 0);
    if (lora && !B) return -1;
    if (!rows) nrows = m;
    if (!cols) ncols = K;
    double u[4096];
    if (r > 4096) return -1;
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t row = rows ? rows[i] : i;
        if (row < 0 || row >= m) return -1;
        const uint16_t *gr = dy + row * N;
        /* u = dy_row . B^T (r values) */
        if (lora) {
            for (int32_t c = 0; c < r; ++c) {
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n)
                    acc += (double)nf4ref_bf16_to_f32(gr[n]) *
                           (double)nf4ref_bf16_to_f32(B[(int64_t)c * N + n]);
                u[c] = acc;
            }
        }
        for (int64_t j = 0; j < ncols; ++j) {
            int64_t col = cols ? cols[j] : j;
            if (col < 0 || col >= K) return -1;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n)
                acc += (double)nf4ref_bf16_to_f32(gr[n]) * (double)wdeq[n * K + col];
            if (lora) {
                double side = 0.0;
                for (int32_t c = 0; c < r; ++c)
                    side += u[c] * (double)nf4ref_bf16_to_f32(A[col * r + c]);
                acc += s * side;
            }
            out[i * ncols + j] = acc;
        }
    }
    return 0;
}

/* [MF] "Gradient Computation": with T = X A and U = dY B^T (m x r, exact in
 * double), dA = s X^T U and dB = s T^T dY, each a plain sum over the m rows. */
int nf4ref_lora_grads(const uint16_t *x, const uint16_t *dy, int64_t m, int64_t K, int64_t N,
                      const uint16_t *A, const uint16_t *B, int32_t r, double s,
                      const int64_t *a_rows, int64_t na, double *da, const int64_t *b_cols,
                      int64_t nb, double *db) {
    if (!x || !dy || !A || !B || m < 0 || K < 0 || N < 0 || r <= 0) return -1;
    if (!a_rows) na = K;
    if (!b_cols) nb = N;
    double *T = (double *)calloc((size_t)(m > 0 ? m : 1) * (size_t)r, sizeof(double));
    double *U = (double *)calloc((size_t)(m > 0 ? m : 1) * (size_t)r, sizeof(double));
    double *acc = (double *)calloc((size_t)r, sizeof(double));
    if (!T || !U || !acc) {
        free(T);
        free(U);
        free(acc);
        return -1;
    }
    for (int64_t i = 0; i < m; ++i) {
        double *t = T + i * r;  /* T[i][c] = sum_k x[i][k] A[k][c] */
        for (int64_t k = 0; k < K; ++k) {
            const double xv = (double)nf4ref_bf16_to_f32(x[i * K + k]);
            for (int32_t c = 0; c < r; ++c) t[c] += xv * (double)nf4ref_bf16_to_f32(A[k * r + c]);
        }
        double *u = U + i * r;  /* U[i][c] = sum_n dy[i][n] B[c][n] */
        for (int32_t c = 0; c < r; ++c) {
            double a = 0.0;
            for (int64_t n = 0; n < N; ++n)
                a += (double)nf4ref_bf16_to_f32(dy[i * N + n]) * (double)nf4ref_bf16_to_f32(B[(int64_t)c * N + n]);
            u[c] = a;
        }
    }
    int rc = 0;
    if (da) {
        for (int64_t j = 0; j < na && rc == 0; ++j) {
            const int64_t k = a_rows ? a_rows[j] : j;
            if (k < 0 || k >= K) {
                rc = -1;
                break;
            }
            for (int32_t c = 0; c < r; ++c) acc[c] = 0.0;
            for (int64_t i = 0; i < m; ++i) {
                const double xv = (double)nf4ref_bf16_to_f32(x[i * K + k]);
                for (int32_t c = 0; c < r; ++c) acc[c] += xv * U[i * r + c];
            }
            for (int32_t c = 0; c < r; ++c) da[j * r + c] = s * acc[c];
        }
    }
    if (db) {
        for (int64_t j = 0; j < nb && rc == 0; ++j) {
            const int64_t n = b_cols ? b_cols[j] : j;
            if (n < 0 || n >= N) {
                rc = -1;
                break;
            }
            for (int32_t c = 0; c < r; ++c) acc[c] = 0.0;
            for (int64_t i = 0; i < m; ++i) {
                const double g = (double)nf4ref_bf16_to_f32(dy[i * N + n]);
                for (int32_t c = 0; c < r; ++c) acc[c] += T[i * r + c] * g;
            }
            for (int32_t c = 0; c < r; ++c) db[c * nb + j] = s * acc[c];
        }
    }
    free(T);
    free(U);
    free(acc);
    return rc;
}

int64_t nf4ref_storage_bytes_ex(int64_t n, int32_t blocksize, int32_t dq_blocksize, int dq,
                                int mean_offset) {
    if (n < 0 || !pow2_in(blocksize, 16, 4096) || !pow2_in(dq_blocksize, 1, 4096)) return -1;
    int64_t nblocks = (n + blocksize - 1) / blocksize;
    int64_t code_bytes = (n + 1) / 2;
    if (!dq) return code_bytes + 4 * nblocks;
    int64_t ngroups = (nblocks + dq_blocksize - 1) / dq_blocksize;
    return code_bytes + nblocks + 4 * ngroups + (mean_offset ? 4 : 0);
}

