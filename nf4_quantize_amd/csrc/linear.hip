// linear.hip - fused NF4-dequant linear for gfx950: forward
//   Y  = X . dequantize(W)^T + s * (X . A) . B
// and input gradient
//   dX = dY . dequantize(W) + s * (dY . B^T) . A^T
// ([MF] "Forward Pass Computation" and "Gradient Computation"; source key in
// nf4_internal.h). W is stored [N x K] row-major with 64-blocks along K.
//
// This file holds the dispatch and the portable tiled path (64x64 output
// tiles, the weight tile dequantized once into LDS and reused by all 64 rows
// of the tile, fp32 FMA), which serves shapes the MFMA paths do not take:
// linear_gemv.hip (m <= 16, no adapter) and linear_gemm.hip (N % 64 == 0,
// r % 8 == 0).
#include "linear_common.h"

namespace nf4 {
namespace {

constexpr int kT = 64;         // output tile edge and K step
constexpr int kThreads = 256;  // 16 x 16 threads, 4 x 4 outputs each

// out[m, j] = sum_i act[m, i] * mat[i * ms_i + j * ms_j]  (bf16 in, fp32 acc,
// bf16 out): the adapter's down-projection X.A (ms_i = r, ms_j = 1) or
// dY.B^T (ms_i = 1, ms_j = N).
__global__ __launch_bounds__(kThreads) void lora_down_simple_kernel(
    const uint16_t *__restrict__ act, int64_t m, int64_t len, const uint16_t *__restrict__ mat,
    int64_t ms_i, int64_t ms_j, int32_t r, uint16_t *__restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= m * r) return;
    const int64_t row = idx / r, j = idx % r;
    float acc = 0.0f;
    for (int64_t i = 0; i < len; ++i)
        acc = fmaf(__uint_as_float((uint32_t)act[row * len + i] << 16),
                   __uint_as_float((uint32_t)mat[i * ms_i + j * ms_j] << 16), acc);
    out[idx] = (uint16_t)(pack_bf16x2(acc, 0.0f) & 0xFFFFu);
}

// kBwd == false: Y tile (rows of X, columns n of W); contraction over K.
// kBwd == true : dX tile (rows of dY, columns k of W); contraction over N.
template <bool kBwd>
__global__ __launch_bounds__(kThreads) void linear_tiled_kernel(
    const uint16_t *__restrict__ act, int64_t m, WView w, const uint16_t *__restrict__ lora_t,
    const uint16_t *__restrict__ lora_mat, int32_t r, float s_lora, uint16_t *__restrict__ out,
    Levels lv) {
    __shared__ float s_a[kT][kT + 1];  // [row][contraction]
    __shared__ float s_w[kT][kT + 1];  // [contraction][output column]
    __shared__ float s_q[16];
    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    if (t < 16) s_q[t] = lv.q[t];
    const int64_t row0 = (int64_t)blockIdx.y * kT;
    const int64_t col0 = (int64_t)blockIdx.x * kT;
    const int64_t ncols = kBwd ? w.k : w.n;   // output width
    const int64_t red = kBwd ? w.n : w.k;     // contraction length
    float acc[4][4] = {};
    for (int64_t c0 = 0; c0 < red; c0 += kT) {
        __syncthreads();
        // activation tile [64 rows x 64 contraction]
        for (int e = t; e < kT * kT; e += kThreads) {
            const int rr = e / kT, cc = e % kT;
            const int64_t gr = row0 + rr, gc = c0 + cc;
            s_a[rr][cc] = (gr < m && gc < red) ? __uint_as_float((uint32_t)act[gr * red + gc] << 16) : 0.0f;
        }
        // weight tile: element (n, k) of W; s_w[contraction][output]
        for (int e = t; e < kT * kT; e += kThreads) {
            const int i0 = e / kT, i1 = e % kT;  // i1 runs along K in memory
            int64_t wn, wk;
            if (kBwd) { wn = c0 + i0; wk = col0 + i1; }
            else      { wn = col0 + i0; wk = c0 + i1; }
            float v = 0.0f;
            if (wn < w.n && wk < w.k) {
                const int64_t idx = wn * w.k + wk;
                const uint32_t code = (w.codes[idx >> 1] >> (4 * (idx & 1))) & 15u;
                v = s_q[code] * wscale(w, idx / kBlock);
            }
            if (kBwd) s_w[i0][i1] = v;   // [n][k]: contraction n, output k
            else      s_w[i1][i0] = v;   // [k][n]: contraction k, output n
        }
        __syncthreads();
#pragma unroll 8
        for (int c = 0; c < kT; ++c) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = s_a[ty * 4 + i][c];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = s_w[c][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
    }
    // adapter side path: + s * sum_t T[row, t] * L[t, col]
    //   forward : L = B [r x N], element (t, n) at t*N + n
    //   backward: L = A^T,       element (t, k) at k*r + t
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t gr = row0 + ty * 4 + i;
        if (gr >= m) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t gc = col0 + tx * 4 + j;
            if (gc >= ncols) continue;
            float v = acc[i][j];
            if (r > 0) {
                float side = 0.0f;
                for (int tt = 0; tt < r; ++tt) {
                    const float tv = __uint_as_float((uint32_t)lora_t[gr * r + tt] << 16);
                    const int64_t li = kBwd ? gc * r + tt : (int64_t)tt * ncols + gc;
                    side = fmaf(tv, __uint_as_float((uint32_t)lora_mat[li] << 16), side);
                }
                v = fmaf(s_lora, side, v);
            }
            out[gr * ncols + gc] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
        }
    }
}

}  // namespace

nf4_linear_path linear_path(int64_t m, int64_t n_out, int64_t k_in, int32_t r, bool backward) {
    if (!backward && r == 0 && gemv_supported(m, k_in)) return NF4_LINEAR_DECODE;
    if (gemm_supported(n_out, r)) return NF4_LINEAR_MFMA;
    return NF4_LINEAR_PORTABLE;
}

hipError_t launch_linear_forward(const uint16_t *x, int64_t m, const nf4_weight &w,
                                 const uint16_t *a, const uint16_t *b, int32_t r, float s_lora,
                                 uint16_t *y, void *workspace, hipStream_t s) {
    const nf4_linear_path path = linear_path(m, w.n_out, w.k_in, r, false);
    if (path == NF4_LINEAR_DECODE) return launch_gemv(x, m, w, y, s);
    if (path == NF4_LINEAR_MFMA)
        return launch_gemm_forward(x, m, w, a, b, r, s_lora, y, static_cast<uint16_t *>(workspace), s);
    uint16_t *t = static_cast<uint16_t *>(workspace);
    if (r > 0)
        lora_down_simple_kernel<<<dim3((unsigned)((m * r + kThreads - 1) / kThreads)), kThreads, 0, s>>>(
            x, m, w.k_in, a, r, 1, r, t);
    dim3 grid((unsigned)((w.n_out + kT - 1) / kT), (unsigned)((m + kT - 1) / kT));
    linear_tiled_kernel<false><<<grid, kThreads, 0, s>>>(x, m, make_view(w), t, b, r, s_lora, y, levels());
    return hipGetLastError();
}

hipError_t launch_linear_backward_input(const uint16_t *dy, int64_t m, const nf4_weight &w,
                                        const uint16_t *a, const uint16_t *b, int32_t r,
                                        float s_lora, uint16_t *dx, void *workspace,
                                        hipStream_t s) {
    if (linear_path(m, w.n_out, w.k_in, r, true) == NF4_LINEAR_MFMA)
        return launch_gemm_dgrad(dy, m, w, a, b, r, s_lora, dx, static_cast<uint16_t *>(workspace), s);
    uint16_t *u = static_cast<uint16_t *>(workspace);
    if (r > 0)
        lora_down_simple_kernel<<<dim3((unsigned)((m * r + kThreads - 1) / kThreads)), kThreads, 0, s>>>(
            dy, m, w.n_out, b, 1, w.n_out, r, u);
    dim3 grid((unsigned)((w.k_in + kT - 1) / kT), (unsigned)((m + kT - 1) / kT));
    linear_tiled_kernel<true><<<grid, kThreads, 0, s>>>(dy, m, make_view(w), u, a, r, s_lora, dx, levels());
    return hipGetLastError();
}

}  // namespace nf4
