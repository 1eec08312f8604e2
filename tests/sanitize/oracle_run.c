/* Runs every function of the CPU oracle (oracle/nf4ref.c) on small and edge
 * case inputs, for the AddressSanitizer / UndefinedBehaviorSanitizer build of
 * tests/test_sanitizers.py. Every buffer is a heap allocation of exactly the
 * size the oracle's header documents, so a read or write one element past it
 * is reported. Results are not checked here (the oracle's pin tests do that),
 * only return codes that the header fixes. Exit status 0: no failure. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "nf4ref.h"

static int failures = 0;
#define EXPECT(cond)                                                              \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond);   \
            ++failures;                                                           \
        }                                                                         \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* splitmix64 -> [0, 1) */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * 0x1p-53;
}
static float gauss(float sigma) {
    double u1 = uniform(), u2 = uniform();
    if (u1 < 1e-300) u1 = 1e-300;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2)) * sigma;
}
static void *xmalloc(size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p) abort();
    return p;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static void storage_path(int64_t n) {
    float *wf = xmalloc((size_t)n * 4);
    uint16_t *wb = xmalloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i) wf[i] = gauss(0.02f);
    if (n > 70) memset(wf + 64, 0, 64 * 4); /* a zero block */
    EXPECT(nf4ref_f32_to_bf16_array(wf, n, wb) == 0);
    const int64_t nb = cdiv(n, 64), ng = cdiv(nb, 256);
    uint8_t *codes = xmalloc((size_t)cdiv(n, 2));
    float *absmax = xmalloc((size_t)nb * 4);
    uint8_t *q = xmalloc((size_t)nb);
    float *scale = xmalloc((size_t)ng * 4);
    float *out = xmalloc((size_t)n * 4);
    uint16_t *outb = xmalloc((size_t)n * 2);
    for (int dt = 0; dt < 2; ++dt) {
        EXPECT(nf4ref_quantize(dt ? (const void *)wb : (const void *)wf, dt, n, codes, absmax) == 0);
        EXPECT(nf4ref_double_quantize(absmax, nb, q, scale) == 0);
        EXPECT(nf4ref_dequantize(codes, n, absmax, NULL, NULL, out, NF4REF_F32) == 0);
        EXPECT(nf4ref_dequantize(codes, n, NULL, q, scale, outb, NF4REF_BF16) == 0);
        if (n > 3) EXPECT(nf4ref_dequantize_range(codes, n, 1, n - 2, NULL, q, scale, out, NF4REF_F32) == 0);
        if (nb > 0) (void)nf4ref_block_scale(nb - 1, absmax, q, scale);
    }
    /* format variants and codebooks */
    const int32_t bss[] = {16, 64, 128, 4096};
    const int32_t dqbs[] = {1, 4, 256, 4096};
    for (int a = 0; a < 4; ++a) {
        const int32_t bs = bss[a];
        const int64_t nbv = cdiv(n, bs);
        float *am = xmalloc((size_t)nbv * 4);
        EXPECT(nf4ref_quantize_bs(wf, NF4REF_F32, n, bs, codes, am) == 0);
        for (int cb = 0; cb < 3; ++cb)
            EXPECT(nf4ref_quantize_cb(wb, NF4REF_BF16, n, bs, cb, codes, am) == 0);
        for (int b = 0; b < 4; ++b)
            for (int fmt = 0; fmt < 3; ++fmt)
                for (int off = 0; off < 2; ++off) {
                    const int32_t dqb = dqbs[b];
                    const int64_t ngv = cdiv(nbv, dqb);
                    uint8_t *qv = xmalloc((size_t)nbv);
                    float *sv = xmalloc((size_t)ngv * 4);
                    float mu = 0.0f;
                    EXPECT(nf4ref_double_quantize_ex(am, nbv, dqb, fmt, off, qv, sv, off ? &mu : NULL) == 0);
                    EXPECT(nf4ref_dequantize_range_ex(codes, n, 0, n, bs, dqb, fmt, NULL, qv, sv,
                                                      off ? &mu : NULL, out, NF4REF_F32) == 0);
                    EXPECT(nf4ref_dequantize_range_cb(codes, n, 0, n, bs, dqb, fmt, NF4REF_CB_FP4, NULL,
                                                      qv, sv, off ? &mu : NULL, outb, NF4REF_BF16) == 0);
                    if (nbv > 0) (void)nf4ref_block_scale_ex(nbv - 1, dqb, fmt, NULL, qv, sv, off ? &mu : NULL);
                    EXPECT(nf4ref_storage_bytes_ex(n, bs, dqb, 1, off) >= 0);
                    free(qv);
                    free(sv);
                }
        free(am);
    }
    EXPECT(nf4ref_storage_bytes(n, 1) >= 0 && nf4ref_storage_bytes(n, 0) >= 0);
    free(wf); free(wb); free(codes); free(absmax); free(q); free(scale); free(out); free(outb);
}

static uint16_t *bf16_gauss(int64_t count, float sigma) {
    uint16_t *p = xmalloc((size_t)count * 2);
    for (int64_t i = 0; i < count; ++i) p[i] = nf4ref_f32_to_bf16(gauss(sigma));
    return p;
}

static void matmuls(int64_t m, int64_t K, int64_t N, int32_t r) {
    uint16_t *x = bf16_gauss(m * K, 1.0f), *dy = bf16_gauss(m * N, 1.0f);
    uint16_t *A = bf16_gauss(K * r, 0.01f), *B = bf16_gauss((int64_t)r * N, 0.01f);
    float *w = xmalloc((size_t)(N * K) * 4);
    for (int64_t i = 0; i < N * K; ++i) w[i] = gauss(0.02f);
    uint8_t *codes = xmalloc((size_t)(N * K / 2));
    const int64_t nb = N * K / 64;
    float *absmax = xmalloc((size_t)nb * 4);
    uint8_t *q = xmalloc((size_t)nb);
    float *scale = xmalloc((size_t)cdiv(nb, 256) * 4);
    EXPECT(nf4ref_quantize(w, NF4REF_F32, N * K, codes, absmax) == 0);
    EXPECT(nf4ref_double_quantize(absmax, nb, q, scale) == 0);
    float *wd = xmalloc((size_t)(N * K) * 4);
    EXPECT(nf4ref_dequantize(codes, N * K, NULL, q, scale, wd, NF4REF_F32) == 0);
    int64_t rows[2] = {0, m - 1}, cols[3] = {0, 1, (N < K ? N : K) - 1};
    double *y = xmalloc((size_t)(m * N) * 8);
    EXPECT(nf4ref_linear_forward(x, m, K, N, wd, A, B, r, 2.0, NULL, 0, NULL, 0, y) == 0);
    EXPECT(nf4ref_linear_forward(x, m, K, N, wd, A, B, r, 2.0, rows, 2, cols, 3, y) == 0);
    double *dx = xmalloc((size_t)(m * K) * 8);
    EXPECT(nf4ref_linear_backward_input(dy, m, K, N, wd, A, B, r, 2.0, NULL, 0, NULL, 0, dx) == 0);
    EXPECT(nf4ref_linear_backward_input(dy, m, K, N, wd, NULL, NULL, 0, 1.0, rows, 2, cols, 3, dx) == 0);
    double *da = xmalloc((size_t)(K * r) * 8), *db = xmalloc((size_t)((int64_t)r * N) * 8);
    EXPECT(nf4ref_lora_grads(x, dy, m, K, N, A, B, r, 2.0, NULL, 0, da, NULL, 0, db) == 0);
    EXPECT(nf4ref_lora_grads(x, dy, m, K, N, A, B, r, 2.0, rows, 2, da, cols, 3, db) == 0);
    float *wm = xmalloc((size_t)(N * K) * 4);
    EXPECT(nf4ref_merged_weight(codes, NULL, q, scale, N, K, A, B, r, 2.0f, NULL, N, wm) == 0);
    EXPECT(nf4ref_merged_weight(codes, absmax, NULL, NULL, N, K, A, B, r, 2.0f, rows, 2, wm) == 0);
    free(x); free(dy); free(A); free(B); free(w); free(codes); free(absmax); free(q); free(scale);
    free(wd); free(y); free(dx); free(da); free(db); free(wm);
}

int main(void) {
    float q[16];
    double c[16];
    nf4ref_codebook(q);
    EXPECT(nf4ref_construct_codebook(0.9677083, c) == 0);
    const double delta = nf4ref_solve_delta((double)q[14]);
    EXPECT(delta > 0.9 && delta < 1.0);
    EXPECT(fabs(nf4ref_normal_quantile(0.5)) < 1e-12);
    for (int cb = 0; cb < 3; ++cb) EXPECT(nf4ref_codebook_levels(cb, q) == 0);
    EXPECT(nf4ref_codebook_levels(3, q) != 0);

    /* element-wise functions over a spread of values, specials included */
    const int64_t nv = 100003;
    float *v = xmalloc((size_t)nv * 4);
    for (int64_t i = 0; i < nv; ++i) v[i] = (float)(uniform() * 2.2 - 1.1);
    v[0] = 0.0f; v[1] = -0.0f; v[2] = 1.0f; v[3] = -1.0f; v[4] = 0x1p-140f; v[5] = 448.0f;
    v[6] = 1e30f; v[7] = -1e30f;
    uint8_t *codes = xmalloc((size_t)nv);
    uint16_t *h = xmalloc((size_t)nv * 2);
    EXPECT(nf4ref_nearest_code_array(v, nv, codes) == 0);
    EXPECT(nf4ref_e4m3_encode_array(v, nv, codes) == 0);
    EXPECT(nf4ref_e5m2_encode_array(v, nv, codes) == 0);
    EXPECT(nf4ref_f32_to_bf16_array(v, nv, h) == 0);
    for (int i = 0; i < 256; ++i) {
        (void)nf4ref_e4m3_decode((uint8_t)i);
        (void)nf4ref_e5m2_decode((uint8_t)i);
        (void)nf4ref_bf16_to_f32((uint16_t)(i << 8 | i));
    }
    for (int64_t n = 0; n < 4100; n += (n < 40 ? 1 : 97)) (void)nf4ref_pairwise_sum(v, n);

    const int64_t sizes[] = {0, 1, 2, 63, 64, 65, 1000, 16383, 16384, 16385, 3 * 16384 + 100};
    for (size_t i = 0; i < sizeof sizes / sizeof sizes[0]; ++i) storage_path(sizes[i]);
    matmuls(5, 128, 64, 8);
    matmuls(17, 192, 320, 16);

    /* non-finite input is rejected, not read past */
    v[10] = NAN;
    float am[2];
    uint8_t cq[32];
    EXPECT(nf4ref_quantize(v, NF4REF_F32, 64, cq, am) != 0);
    EXPECT(nf4ref_storage_bytes(-1, 1) < 0);
    free(v); free(codes); free(h);
    if (failures) fprintf(stderr, "%d failures\n", failures);
    else printf("oracle sanitizer run: ok\n");
    return failures ? 1 : 0;
}
