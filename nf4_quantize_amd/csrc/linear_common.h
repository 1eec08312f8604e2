// linear_common.h - weight view and level table shared by the fused NF4
// linear kernels (internal).
#pragma once

#include <algorithm>

#include "nf4_internal.h"

namespace nf4 {

// An NF4 weight [n x k] (row-major, 64-blocks along k) as passed to kernels.
struct WView {
    const uint8_t *codes;
    const uint8_t *q;      // E4M3 codes of c1/c2, or nullptr
    const float *scale;    // c2 per group (with q)
    const float *absmax;   // c1 per block (without q)
    int64_t n, k;
};

inline WView make_view(const nf4_weight &w) {
    return WView{w.codes, w.absmax_q, w.absmax_scale, w.absmax, w.n_out, w.k_in};
}

// Reconstructed scale c1' of flat block index b.
__device__ __forceinline__ float wscale(const WView &w, int64_t b) {
    return block_scale(b, w.absmax, w.q, w.scale);
}

// The 16 levels by value (kernel argument).
struct Levels {
    float q[16];
};
inline Levels levels() {
    Levels l;
    for (int i = 0; i < 16; ++i) l.q[i] = kLevels[i];
    return l;
}

// Decode-shaped path (1 <= m <= 16, K % 256 == 0, no adapter): linear_gemv.hip.
bool gemv_supported(int64_t m, int64_t k);
hipError_t launch_gemv(const uint16_t *x, int64_t m, const nf4_weight &w, uint16_t *y,
                       hipStream_t s);

// Adapter workspace: the bf16 product [m x rp] (rp = r rounded up to 64),
// padded to 256 bytes, then room for kSplitMax fp32 partial sums of it.
constexpr int kSplitMax = 8;
inline size_t lora_product_bytes(int64_t m, int64_t rp) { return ((size_t)(m * rp * 2) + 255u) & ~(size_t)255u; }
inline size_t lora_workspace_bytes(int64_t m, int64_t rp) {
    return lora_product_bytes(m, rp) + (size_t)kSplitMax * (size_t)(m * rp) * 4u;
}

// Adapter down-projection C[m x rp] = scale * Aop . Bop^T (linear_adapter.hip):
// Bop[c][k] = mat[k][c] (nn: A [klen x r], ldm = r) or mat[c][k] (B [r x ldm]).
// With partial != nullptr, split z of `splits` writes its fp32 sum to
// partial[z][m][rp] instead of c. Needs r % 8 == 0 and rp % 64 == 0.
bool adapter_down_supported(bool nn, int64_t lda, int64_t klen, int64_t ldm, int32_t r);
hipError_t launch_adapter_down(bool nn, const uint16_t *aop, int64_t lda, int64_t m, int64_t klen,
                               const uint16_t *mat, int64_t ldm, int32_t r, int64_t rp, int splits,
                               float *partial, uint16_t *c, float scale, hipStream_t s);
// Both down-projections of the adapter gradients in one launch: T = X.A
// (fwd, the forward form) and U = dY.B^T (bwd), each with its own split count
// and partial area (nullptr when not split).
struct DownJob {
    const uint16_t *aop;
    int64_t lda, klen;
    const uint16_t *mat;
    int64_t ldm;
    int splits;
    float *partial;
    uint16_t *c;
};
hipError_t launch_adapter_down_pair(const DownJob &fwd, const DownJob &bwd, int64_t m, int32_t r, int64_t rp,
                                    float scale, hipStream_t s);

// Token sums of the adapter gradients (linear_adapter.hip): C[o][j] =
// sum over the m tokens of P[t][o] * Q[t][j], P [m x O] (O % 64 == 0),
// Q [m x rp] bf16 (columns past r unused). With partial != nullptr split z of
// `splits` writes its fp32 sum to partial[z] ([O x r], or [r x O] when
// transposed); otherwise scale * C goes to out (fp32 or bf16, [O x r] or
// [r x O]). The paired launch can take Q transposed instead: Q^T [rp x qt]
// bf16, row j holding Q[t][j] at t (qt = lora_qt_row(m), zeros past m).
bool token_sum_supported(int64_t m, int64_t O, int64_t rp);
hipError_t launch_token_sum(const uint16_t *pm, const uint16_t *qm, int64_t m, int64_t O, int64_t rp, int32_t r,
                            int splits, float *partial, void *out, bool f32, bool transposed, float scale,
                            hipStream_t s);
// Two token sums in one launch (dA and dB), each with its own split count and
// partial area (nullptr when not split: then scale * C goes to out).
struct TokenSumJob {
    const uint16_t *pm, *qm;
    int64_t O;
    bool transposed;
    int splits;
    float *partial;
    void *out;
};
// qt: 0 for Q [m x rp], else the row length of Q^T [rp x qt] (both jobs).
hipError_t launch_token_sum_pair(const TokenSumJob &a, const TokenSumJob &b, int64_t m, int64_t rp, int32_t r,
                                 bool f32, float scale, int64_t qt, hipStream_t s);
// Row length (tokens) of the transposed Q of the paired token sums: m
// rounded up to whole 64-token steps, plus one more 128-byte line, so that
// rows do not sit a power of two apart (every workgroup reads the same 64
// rows per step; with a 2^k-byte row stride they shared one L2 channel).
inline int64_t lora_qt_row(int64_t m) { return (m + 63) / 64 * 64 + 64; }
// The transposed Q fits 32-bit buffer offsets.
inline bool token_sum_qt_supported(int64_t m, int64_t rp) { return rp * lora_qt_row(m) * 2 < ((int64_t)1 << 31); }

// Large-M MFMA path (N % 64 == 0, r % 8 == 0, r <= 256): linear_gemm.hip.
bool gemm_supported(int64_t n, int32_t r);
hipError_t launch_gemm_forward(const uint16_t *x, int64_t m, const nf4_weight &w, const uint16_t *a,
                               const uint16_t *b, int32_t r, float s_lora, uint16_t *y,
                               uint16_t *t_ws, hipStream_t s);
hipError_t launch_gemm_dgrad(const uint16_t *dy, int64_t m, const nf4_weight &w, const uint16_t *a,
                             const uint16_t *b, int32_t r, float s_lora, uint16_t *dx,
                             uint16_t *u_ws, hipStream_t s);

// Adapter gradients dA = s X^T (dY B^T) [K x r] and dB = s (X A)^T dY [r x N]
// (linear_gemm.hip); da or db may be nullptr. Needs K % 64 == 0, N % 64 == 0,
// r % 8 == 0, r <= 256, and a workspace of lora_grads_workspace_bytes.
// Layout: T and U (bf16, lora_product_bytes of lora_qt_row(m) tokens each:
// the token sums read them transposed and zero-padded), then the fp32
// partial sums of both down-projections, later of both token sums.
inline size_t lora_grads_workspace_bytes(int64_t m, int64_t k, int64_t n, int64_t rp, int64_t r) {
    const int64_t most = std::max(2 * m * rp, k * r + r * n);
    return 2 * lora_product_bytes(lora_qt_row(m), rp) + (size_t)kSplitMax * (size_t)most * 4u;
}
hipError_t launch_lora_grads(const uint16_t *x, const uint16_t *dy, int64_t m, int64_t K, int64_t N,
                             const uint16_t *a, const uint16_t *b, int32_t r, float s_lora, void *da, void *db,
                             bool f32_out, void *ws, hipStream_t s);

// Main forward GEMM of the large-M path (linear_fwd.hip): Y = X . W'^T, plus
// T' . B when t != nullptr (T' bf16 [m x rp]). Needs K <= 2^22.
bool fwd_main_supported(int64_t k);
hipError_t launch_fwd_main(const uint16_t *x, int64_t m, const nf4_weight &w, const uint16_t *t,
                           int64_t rp, const uint16_t *b, int32_t r, uint16_t *y, hipStream_t s);

// Main input-gradient GEMM of the large-M path (linear_dgrad.hip): dX = dY . W',
// plus U' . A^T when u != nullptr. Needs N * K / 2 < 2^31.
bool dgrad_main_supported(int64_t n, int64_t k);
hipError_t launch_dgrad_main(const uint16_t *dy, int64_t m, const nf4_weight &w, const uint16_t *u,
                             int64_t rp, const uint16_t *a, int32_t r, uint16_t *dx, hipStream_t s);

}  // namespace nf4
