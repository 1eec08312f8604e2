// linear_gemm.hip - large-M fused NF4 linear for gfx950 on bf16 MFMA
// ([MF] "Forward Pass Computation" and "Gradient Computation"; source key in
// nf4_internal.h):
//   forward   Y  = X . W'^T + s (X . A) . B
//   dgrad     dX = dY . W'  + s (dY . B^T) . A^T
// with W' = dequantize(W), W stored [N x K] NF4, A [K x r], B [r x N] bf16.
//
// One kernel template computes C[M x Nc] = sum over K-segments of
// Aop[M x Kseg] . Bop[Nc x Kseg]^T, where Aop is a row-major bf16 matrix and
// Bop is read from one of four sources:
//   NF4_NT  Bop[n][k] = W'[n][k]   (forward: rows of W)
//   NF4_NN  Bop[c][j] = W'[j][c]   (dgrad: columns of W)
//   BF16_NT Bop[n][k] = Mat[n][k]
//   BF16_NN Bop[n][k] = Mat[k][n]
// A second K-segment carries the adapter: forward appends T' = s X.A with
// Bop = B (BF16_NN), dgrad appends U' = s dY.B^T with Bop = A (BF16_NT);
// T' and U' come from the same kernel (BF16_NN with Mat = A, and BF16_NT
// with Mat = B) and are stored bf16 in the caller's workspace.
//
// Tiling: a workgroup of 4 waves owns a BM x BN tile of C; each wave a
// (BM/2) x (BN/2) quarter, as 16x16 tiles of v_mfma_f32_16x16x32_bf16.
// K advances 64 at a time (one NF4 block per weight row). Both operand tiles
// are staged in LDS as bf16 [row][64] with 16-byte chunks XOR-swizzled by row
// so that the MFMA operand reads (16 rows, one chunk) hit distinct banks.
// The NF4 tile is dequantized on the way in, exactly as the dequantize path
// does it: bf16(q[code] * c1'). The next K-step's global loads are issued
// before the current step's MFMAs; LDS is double buffered.
#include <algorithm>
#include <type_traits>

#include "linear_common.h"

namespace nf4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBK = 64;           // K step (one NF4 block per weight row)
constexpr int kRowBytes = kBK * 2;

enum BMode { NF4_NT = 0, NF4_NN = 1, BF16_NT = 2, BF16_NN = 3 };

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS tile row `row`.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return (uint32_t)row * kRowBytes + 16u * (uint32_t)(chunk ^ ((row >> 1) & 7));
}

// One K-segment: C += Aop . Bop^T over ksteps of 64.
struct Segment {
    const uint16_t *a;   // Aop, row-major [M x lda] (transposed A: [a_krows x lda], Aop[i][k] = a[k][i])
    int64_t lda;
    int64_t klen;        // contraction length of the segment (multiple of 64)
    int64_t a_krows;     // transposed A: rows of a (contraction values past it read as zero)
    // B source
    WView w;             // NF4 modes
    const uint16_t *mat; // bf16 modes
    int64_t ldm;         // row stride of mat
    int64_t mat_rows, mat_cols;  // bounds of mat
};

struct Params {
    Segment seg[2];
    int nseg;
    int64_t M, Nc;       // C is [M x Nc]
    uint16_t *c;         // bf16 output
    int64_t ldc;
    float out_scale;     // multiplies the fp32 accumulator before rounding
    Levels lv;
    // split-K (grid.y = splits): when partial != nullptr, split z writes its
    // unscaled fp32 sum to partial[(z * M + row) * ldc + col] instead of c.
    int splits;
    float *partial;
};

// ---------------------------------------------------------------- staging

// A tile: BM rows x 64 bf16 = BM * 8 chunks; each thread moves BM/32 chunks.
template <int BM>
struct AStage {
    static constexpr int kChunks = BM * 8 / kThreads;
    u32x4 v[kChunks];
    __device__ void load(const Segment &sg, int64_t m0, int64_t M, int64_t k0) {
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const int idx = q * kThreads + threadIdx.x;
            const int row = idx >> 3, ch = idx & 7;
            const int64_t gr = m0 + row;
            v[q] = u32x4{0, 0, 0, 0};
            if (gr < M) v[q] = *reinterpret_cast<const u32x4 *>(sg.a + gr * sg.lda + k0 + ch * 8);
        }
    }
    __device__ void store(char *lds) const {
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const int idx = q * kThreads + threadIdx.x;
            *reinterpret_cast<u32x4 *>(lds + swz(idx >> 3, idx & 7)) = v[q];
        }
    }
};

// 8x8 bf16 transpose within a thread: in[i] holds row i (8 values as 4
// dwords), out[j] holds column j.
__device__ __forceinline__ void transpose8x8(const u32x4 (&in)[8], u32x4 (&out)[8]) {
    // element (i, j) is the 16-bit half (j & 1) of dword j >> 1 of in[i]
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = in[2 * p][j >> 1], hi = in[2 * p + 1][j >> 1];
            // pick half (j & 1) of lo and of hi into one dword (lo half first)
            d[p] = (j & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                           : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        out[j] = u32x4{d[0], d[1], d[2], d[3]};
    }
}

// A tile read across rows: Aop[i][k] = a[k][i] for BM rows i and 64
// contraction values k (the token sums of the adapter gradients). Thread t
// owns an 8 (k) x 8 (i) patch, loaded as 8 row pieces and transposed in
// registers; needs M % 8 == 0 and lda % 8 == 0.
template <int BM>
struct AStageT {
    static constexpr int kPatches = BM * kBK / 64;  // threads beyond this idle
    static_assert(kPatches <= kThreads, "at most one 8x8 patch per thread");
    u32x4 r[8];
    __device__ void load(const Segment &sg, int64_t m0, int64_t M, int64_t k0) {
        const int t = threadIdx.x;
        if (t >= kPatches) return;
        const int kp = t & 7, ip = t >> 3;
        const int64_t i = m0 + ip * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t k = k0 + kp * 8 + e;
            r[e] = u32x4{0, 0, 0, 0};
            if (k < sg.a_krows && i < M) r[e] = *reinterpret_cast<const u32x4 *>(sg.a + k * sg.lda + i);
        }
    }
    __device__ void store(char *lds) const;
};

template <int BM>
__device__ void AStageT<BM>::store(char *lds) const {
    const int t = threadIdx.x;
    if (t >= kPatches) return;
    const int kp = t & 7, ip = t >> 3;
    u32x4 cols[8];
    transpose8x8(r, cols);
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(lds + swz(ip * 8 + j, kp)) = cols[j];
}

// B tile, NF4 read along K (forward): BN weight rows x one 64-block.
// Thread t owns row t % BN's block part: BN/64 ... for BN = 256 one full
// block (64 weights); for BN = 64 a quarter block (16 weights).
template <int BN>
struct BStageNF4NT {
    static constexpr int kW = BN * kBK / kThreads;  // weights per thread (64 or 16)
    static constexpr int kParts = kBK / kW;         // threads per row
    u32x4 c[kW / 32 > 0 ? kW / 32 : 1];             // packed codes (16 B = 32 weights)
    uint32_t cw;                                    // 8 B case: codes of 16 weights
    float sc;
    __device__ void load(const Segment &sg, int64_t n0, int64_t Nc, int64_t k0) {
        const int t = threadIdx.x;
        const int row = t / kParts, part = t % kParts;
        const int64_t n = n0 + row;
        sc = 0.0f;
        if (kW == 64) {
            c[0] = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
            c[1] = c[0];
        } else {
            cw = 0x77777777u;
        }
        uint64_t cw2 = 0x7777777777777777ull;
        if (n < Nc) {
            const uint8_t *p = sg.w.codes + (uint64_t)n * ((uint64_t)sg.w.k / 2) + (uint64_t)k0 / 2 + part * (kW / 2);
            if (kW == 64) {
                c[0] = reinterpret_cast<const u32x4 *>(p)[0];
                c[1] = reinterpret_cast<const u32x4 *>(p)[1];
            } else {
                cw2 = *reinterpret_cast<const uint64_t *>(p);
            }
            sc = wscale(sg.w, n * (sg.w.k / kBlock) + k0 / kBlock);
        }
        if (kW != 64) {
            c[0] = u32x4{(uint32_t)cw2, (uint32_t)(cw2 >> 32), 0, 0};
        }
    }
    __device__ void store(char *lds, const float *s_q) const {
        const int t = threadIdx.x;
        const int row = t / kParts, part = t % kParts;
        constexpr int kDw = kW / 8;  // code dwords (8 weights each)
#pragma unroll
        for (int d = 0; d < kDw; ++d) {
            const uint32_t cd = c[d / 4][d % 4];
            u32x4 o;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t b = (cd >> (8 * h)) & 0xFFu;
                o[h] = pack_bf16x2(s_q[b & 15] * sc, s_q[b >> 4] * sc);
            }
            *reinterpret_cast<u32x4 *>(lds + swz(row, part * kDw + d)) = o;
        }
    }
};

// B tile, NF4 read across rows (dgrad): Bop[c][j] = W'[j][c] for 64 rows j
// and BN columns c. Thread t owns an 8 (j) x 8 (c) patch.
template <int BN>
struct BStageNF4NN {
    static constexpr int kPatches = BN * kBK / 64;  // threads beyond this idle
    static_assert(kPatches <= kThreads, "at most one 8x8 patch per thread");
    uint32_t cd[8];  // codes of 8 rows j, 8 columns c (one dword each)
    float sc[8];
    __device__ void load(const Segment &sg, int64_t c0, int64_t Nc, int64_t j0) {
        const int t = threadIdx.x;
        if (t >= kPatches) return;
        const int jp = t & 7, cp = t >> 3;  // j patch 0..7, c patch 0..BN/8-1
        const int64_t cc = c0 + cp * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t j = j0 + jp * 8 + i;  // weight row
            cd[i] = 0x77777777u;
            sc[i] = 0.0f;
            if (cc < Nc) {  // Nc = K of W, a multiple of 64, so cc + 7 < Nc
                cd[i] = *reinterpret_cast<const uint32_t *>(sg.w.codes + (uint64_t)j * ((uint64_t)sg.w.k / 2) + (uint64_t)cc / 2);
                sc[i] = wscale(sg.w, j * (sg.w.k / kBlock) + cc / kBlock);
            }
        }
    }
    __device__ void store(char *lds, const float *s_q) const {
        const int t = threadIdx.x;
        if (t >= kPatches) return;
        const int jp = t & 7, cp = t >> 3;
        u32x4 rows[8], cols[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const uint32_t b = (cd[i] >> (8 * h)) & 0xFFu;
                rows[i][h] = pack_bf16x2(s_q[b & 15] * sc[i], s_q[b >> 4] * sc[i]);
            }
        }
        transpose8x8(rows, cols);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(lds + swz(cp * 8 + j, jp)) = cols[j];
    }
};

// B tile, bf16 Bop[n][k] = Mat[n][k] (rows of Mat): like the A tile.
template <int BN>
struct BStageBF16NT {
    static constexpr int kChunks = BN * 8 / kThreads;
    u32x4 v[kChunks];
    __device__ void load(const Segment &sg, int64_t n0, int64_t Nc, int64_t k0) {
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const int idx = q * kThreads + threadIdx.x;
            const int row = idx >> 3, ch = idx & 7;
            const int64_t n = n0 + row, k = k0 + ch * 8;
            v[q] = u32x4{0, 0, 0, 0};
            if (n < sg.mat_rows && k < sg.mat_cols)  // mat_cols is a multiple of 8
                v[q] = *reinterpret_cast<const u32x4 *>(sg.mat + n * sg.ldm + k);
        }
    }
    __device__ void store(char *lds, const float *) const {
#pragma unroll
        for (int q = 0; q < kChunks; ++q) {
            const int idx = q * kThreads + threadIdx.x;
            *reinterpret_cast<u32x4 *>(lds + swz(idx >> 3, idx & 7)) = v[q];
        }
    }
};

// B tile, bf16 Bop[n][k] = Mat[k][n] (columns of Mat): 8x8 patches.
template <int BN>
struct BStageBF16NN {
    static constexpr int kPatches = BN * kBK / 64;  // threads beyond this idle
    static_assert(kPatches <= kThreads, "at most one 8x8 patch per thread");
    u32x4 r[8];
    __device__ void load(const Segment &sg, int64_t n0, int64_t Nc, int64_t k0) {
        const int t = threadIdx.x;
        if (t >= kPatches) return;
        const int kp = t & 7, np = t >> 3;
        const int64_t n = n0 + np * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t k = k0 + kp * 8 + i;
            r[i] = u32x4{0, 0, 0, 0};
            if (k < sg.mat_rows && n < sg.mat_cols)  // mat_cols is a multiple of 8
                r[i] = *reinterpret_cast<const u32x4 *>(sg.mat + k * sg.ldm + n);
        }
    }
    __device__ void store(char *lds, const float *) const {
        const int t = threadIdx.x;
        if (t >= kPatches) return;
        const int kp = t & 7, np = t >> 3;
        u32x4 cols[8];
        transpose8x8(r, cols);
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<u32x4 *>(lds + swz(np * 8 + j, kp)) = cols[j];
    }
};

template <int Mode, int BN> struct BStageOf;
template <int BN> struct BStageOf<NF4_NT, BN> { using T = BStageNF4NT<BN>; };
template <int BN> struct BStageOf<NF4_NN, BN> { using T = BStageNF4NN<BN>; };
template <int BN> struct BStageOf<BF16_NT, BN> { using T = BStageBF16NT<BN>; };
template <int BN> struct BStageOf<BF16_NN, BN> { using T = BStageBF16NN<BN>; };

// ---------------------------------------------------------------- kernel

// Tile index -> (m tile, n tile): consecutive workgroups go to different XCDs
// (round robin over 8), so each XCD is given a contiguous run of tiles, taken
// n-group-major (4 n tiles x all m tiles) so that its concurrent workgroups
// share operand rows in its L2.
__device__ __forceinline__ void tile_coords(int64_t wg, int64_t tm, int64_t tn, int64_t &mt, int64_t &nt) {
    const int64_t total = tm * tn;
    // a bijection only when total is a multiple of 8; otherwise keep the order
    const int64_t L = (total % 8 == 0) ? (wg % 8) * (total / 8) + wg / 8 : wg;
    const int64_t gn = 4;
    const int64_t group = L / (gn * tm);
    const int64_t within = L % (gn * tm);
    const int64_t ncols = min(gn, tn - group * gn);
    mt = within / ncols;
    nt = group * gn + within % ncols;
}

template <int BM, int BN, int Mode0, int Mode1, bool kAT = false>
__global__ __launch_bounds__(kThreads) void gemm_kernel(Params p) {
    constexpr int WM = BM / 2, WN = BN / 2;   // wave tile
    constexpr int TM = WM / 16, TN = WN / 16; // 16x16 MFMA tiles per wave
    constexpr int kABytes = BM * kRowBytes, kBBytes = BN * kRowBytes;
    extern __shared__ __align__(16) char smem[];
    // LDS: A buffers 0/1, then B buffers 0/1, then the 16 levels
    char *const sA0 = smem;
    char *const sB0 = smem + 2 * kABytes;
    float *const s_q = reinterpret_cast<float *>(smem + 2 * (kABytes + kBBytes));

    if (threadIdx.x < 16) s_q[threadIdx.x] = p.lv.q[threadIdx.x];

    const int64_t tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.Nc + BN - 1) / BN;
    int64_t mt, nt;
    tile_coords(blockIdx.x, tiles_m, tiles_n, mt, nt);
    const int64_t m0 = mt * BM, n0 = nt * BN;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
    const int g = lane >> 4, r = lane & 15;

    f32x4_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t steps0 = p.seg[0].klen / kBK;
    const int64_t steps = steps0 + (p.nseg > 1 ? p.seg[1].klen / kBK : 0);

    using B0 = typename BStageOf<Mode0, BN>::T;
    using B1 = typename BStageOf<Mode1, BN>::T;
    std::conditional_t<kAT, AStageT<BM>, AStage<BM>> ra;
    B0 rb0;
    B1 rb1;

    auto load = [&](int64_t s) {
        if (s < steps0) {
            ra.load(p.seg[0], m0, p.M, s * kBK);
            rb0.load(p.seg[0], n0, p.Nc, s * kBK);
        } else {
            ra.load(p.seg[1], m0, p.M, (s - steps0) * kBK);
            rb1.load(p.seg[1], n0, p.Nc, (s - steps0) * kBK);
        }
    };
    auto store = [&](int64_t s, int buf) {
        ra.store(sA0 + buf * kABytes);
        if (s < steps0)
            rb0.store(sB0 + buf * kBBytes, s_q);
        else
            rb1.store(sB0 + buf * kBBytes, s_q);
    };

    // this workgroup's share of the K-steps (all of them without split-K;
    // only the small-tile instantiations of the adapter products split K)
    constexpr bool kSplit = (BM == 64);
    const int64_t per = kSplit ? (steps + p.splits - 1) / p.splits : steps;
    const int64_t s_lo = kSplit ? min(steps, (int64_t)blockIdx.y * per) : 0;
    const int64_t s_hi = kSplit ? min(steps, s_lo + per) : steps;

    __syncthreads();  // s_q
    if (s_lo < s_hi) {
        load(s_lo);
        store(s_lo, 0);
    }
    __syncthreads();
    for (int64_t s = s_lo; s < s_hi; ++s) {
        const int buf = (s - s_lo) & 1;
        const char *const a_t = sA0 + buf * kABytes;
        const char *const b_t = sB0 + buf * kBBytes;
        if (s + 1 < s_hi) load(s + 1);
        // MFMAs of step s from LDS buffer buf
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 af[TM], bfr[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = *reinterpret_cast<const u32x4 *>(a_t + swz(wm + 16 * i + r, ks * 4 + g));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bfr[j] = *reinterpret_cast<const u32x4 *>(b_t + swz(wn + 16 * j + r, ks * 4 + g));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[i]), as_bf16x8(bfr[j]),
                                                                        acc[i][j], 0, 0, 0);
        }
        if (s + 1 < s_hi) store(s + 1, buf ^ 1);
        __syncthreads();
    }

    // epilogue: D row 4 g + q, column r of each 16x16 tile
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = n0 + wn + 16 * j + r;
            if (col >= p.Nc) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = m0 + wm + 16 * i + 4 * g + q;
                if (row >= p.M) continue;
                if (kSplit && p.partial)
                    p.partial[((int64_t)blockIdx.y * p.M + row) * p.ldc + col] = acc[i][j][q];
                else
                    p.c[row * p.ldc + col] = (uint16_t)(pack_bf16x2(acc[i][j][q] * p.out_scale, 0.0f) & 0xFFFFu);
            }
        }
}

template <int BM, int BN, int Mode0, int Mode1, bool kAT = false>
hipError_t run(const Params &p_in, hipStream_t s) {
    Params p = p_in;
    p.splits = max(1, p.splits);
    const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.Nc + BN - 1) / BN);
    const size_t lds = 2 * (size_t)(BM + BN) * kRowBytes + 64;
    auto kern = gemm_kernel<BM, BN, Mode0, Mode1, kAT>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)tiles, (unsigned)max(1, p.splits)), dim3(kThreads), lds, s>>>(p);
    return hipGetLastError();
}

Segment nf4_segment(const uint16_t *a, int64_t lda, int64_t klen, const WView &w) {
    Segment sg{};
    sg.a = a;
    sg.lda = lda;
    sg.klen = klen;
    sg.w = w;
    return sg;
}

Segment bf16_segment(const uint16_t *a, int64_t lda, int64_t klen, const uint16_t *mat, int64_t ldm,
                     int64_t rows, int64_t cols) {
    Segment sg{};
    sg.a = a;
    sg.lda = lda;
    sg.klen = klen;
    sg.mat = mat;
    sg.ldm = ldm;
    sg.mat_rows = rows;
    sg.mat_cols = cols;
    return sg;
}

int64_t round64(int64_t v) { return (v + 63) / 64 * 64; }

// out[i] = scale * sum over z of part[z * count + i], rounded to bf16 or kept
// fp32, 4 elements per thread (count is a multiple of 4).
template <bool kF32>
__device__ __forceinline__ void reduce_partials_at(const float *__restrict__ part, int splits, int64_t count,
                                                   float scale, void *__restrict__ out, int64_t i) {
    if (i >= count) return;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(part + i);
    for (int z = 1; z < splits; ++z) acc += *reinterpret_cast<const f32x4 *>(part + z * count + i);
    if constexpr (kF32) {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + i) = acc * scale;
    } else {
        uint2 o;
        o.x = pack_bf16x2(scale * acc[0], scale * acc[1]);
        o.y = pack_bf16x2(scale * acc[2], scale * acc[3]);
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(out) + i) = o;
    }
}

template <bool kF32 = false>
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float *__restrict__ part, int splits,
                                                              int64_t count, float scale, void *__restrict__ out) {
    reduce_partials_at<kF32>(part, splits, count, scale, out, ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4);
}

// Two such passes in one launch: workgroups below b1 take job a, the others job b.
struct ReduceJob {
    const float *part;
    int splits;
    int64_t count;  // 0: nothing to add
    void *out;
};
template <bool kF32>
__global__ __launch_bounds__(256) void reduce_partials_pair_kernel(ReduceJob a, ReduceJob b, int64_t b1,
                                                                   float scale) {
    const bool second = (int64_t)blockIdx.x >= b1;
    const ReduceJob &j = second ? b : a;
    const int64_t blk = second ? (int64_t)blockIdx.x - b1 : (int64_t)blockIdx.x;
    reduce_partials_at<kF32>(j.part, j.splits, j.count, scale, j.out, (blk * 256 + threadIdx.x) * 4);
}
// The split sums of a down-projection written transposed, for the token
// sums: out[j][t] = bf16(scale * sum_z part[z][t][j]) (the sum in the order
// of reduce_partials_at, so the values are those of the row-major pass), with
// zeros for tokens m <= t < ld and columns j >= r (ld: lora_qt_row(m)).
// A workgroup owns 32 tokens x 64 columns and turns them around in LDS (row
// stride 65 floats: both the row writes and the column reads hit distinct
// banks).
struct TransposeJob {
    const float *part;  // [splits][m][rp] fp32
    int splits;
    int64_t m, rp, ld;
    int32_t r;
    uint16_t *out;      // [rp][ld] bf16
};
__global__ __launch_bounds__(256) void reduce_transpose_pair_kernel(TransposeJob a, TransposeJob b, int64_t b1,
                                                                    float scale) {
    __shared__ float s_t[32][65];
    const bool second = (int64_t)blockIdx.x >= b1;
    const TransposeJob &J = second ? b : a;
    const int64_t blk = second ? (int64_t)blockIdx.x - b1 : (int64_t)blockIdx.x;
    const int64_t tiles_t = J.ld / 32;
    const int64_t t0 = (blk % tiles_t) * 32, j0 = (blk / tiles_t) * 64;
    const int tid = threadIdx.x;
    const int cc = 4 * (tid & 15);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int rr = (tid >> 4) + 16 * k;
        const int64_t t = t0 + rr;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        if (t < J.m) {
            const float *src = J.part + t * J.rp + j0 + cc;
            acc = *reinterpret_cast<const f32x4 *>(src);
            for (int z = 1; z < J.splits; ++z) acc += *reinterpret_cast<const f32x4 *>(src + z * J.m * J.rp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) s_t[rr][cc + e] = (j0 + cc + e < J.r) ? scale * acc[e] : 0.0f;
    }
    __syncthreads();
    // thread: column j0 + tid / 4, tokens t0 + 8 (tid % 4) .. +7 (one 16-byte store)
    const int jj = tid >> 2, tq = 8 * (tid & 3);
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w4[e] = pack_bf16x2(s_t[tq + 2 * e][jj], s_t[tq + 2 * e + 1][jj]);
    *reinterpret_cast<u32x4 *>(J.out + (j0 + jj) * J.ld + t0 + tq) = u32x4{w4[0], w4[1], w4[2], w4[3]};
}
hipError_t reduce_transpose_pair(const TransposeJob &a, const TransposeJob &b, float scale, hipStream_t s) {
    const int64_t ba = (a.ld / 32) * (a.rp / 64), bb = (b.ld / 32) * (b.rp / 64);
    if (ba + bb == 0) return hipSuccess;
    reduce_transpose_pair_kernel<<<dim3((unsigned)(ba + bb)), 256, 0, s>>>(a, b, ba, scale);
    return hipGetLastError();
}

hipError_t reduce_pair(bool f32, const ReduceJob &a, const ReduceJob &b, float scale, hipStream_t s) {
    const int64_t ba = (a.count / 4 + 255) / 256, bb = (b.count / 4 + 255) / 256;
    if (ba + bb == 0) return hipSuccess;
    if (f32)
        reduce_partials_pair_kernel<true><<<dim3((unsigned)(ba + bb)), 256, 0, s>>>(a, b, ba, scale);
    else
        reduce_partials_pair_kernel<false><<<dim3((unsigned)(ba + bb)), 256, 0, s>>>(a, b, ba, scale);
    return hipGetLastError();
}

// Adapter down-projection C[m x rp] = s * Aop . Bop^T (bf16) into the start of
// the workspace. The product is thin (rp columns) and long (klen), so K is
// split across workgroups to fill the chip; the fp32 partial sums go to the
// workspace after C and one more pass adds, scales and rounds them.
template <int Mode>
hipError_t lora_down(const Segment &sg, int64_t m, int64_t rp, float s_lora, uint16_t *ws, const Levels &lv,
                     hipStream_t s, float *partial_area = nullptr) {
    Params q{};
    q.lv = lv;
    q.seg[0] = sg;
    q.nseg = 1;
    q.M = m;
    q.Nc = rp;
    q.c = ws;
    q.ldc = rp;
    q.out_scale = s_lora;
    const int64_t tiles = ((m + 63) / 64) * (rp / 64), steps = sg.klen / kBK;
    int splits = (int)min((int64_t)kSplitMax, max((int64_t)1, (512 + tiles - 1) / tiles));
    splits = (int)min((int64_t)splits, max((int64_t)1, steps));
    q.splits = splits;
    if (!partial_area) partial_area = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + lora_product_bytes(m, rp));
    float *const partial = splits > 1 ? partial_area : nullptr;
    // the streaming kernel of linear_adapter.hip; the generic one otherwise
    constexpr bool kNN = (Mode == BF16_NN);
    const int32_t r = (int32_t)(kNN ? sg.mat_cols : sg.mat_rows);
    hipError_t e;
    if (adapter_down_supported(kNN, sg.lda, sg.klen, sg.ldm, r)) {
        e = launch_adapter_down(kNN, sg.a, sg.lda, m, sg.klen, sg.mat, sg.ldm, r, rp, splits, partial, ws,
                                s_lora, s);
        if (e != hipSuccess || splits == 1) return e;
    } else {
        if (splits == 1) return run<64, 64, Mode, Mode>(q, s);
        q.partial = partial;
        e = run<64, 64, Mode, Mode>(q, s);
        if (e != hipSuccess) return e;
    }
    const int64_t count = m * rp;
    reduce_partials_kernel<<<dim3((unsigned)((count / 4 + 255) / 256)), 256, 0, s>>>(partial, splits, count,
                                                                                     s_lora, ws);
    return hipGetLastError();
}

}  // namespace

bool gemm_supported(int64_t n, int32_t r) { return n % 64 == 0 && r % 8 == 0 && r <= 256; }

// Forward: T' = s X.A (when r > 0), then Y = X.W'^T + T'.B.
hipError_t launch_gemm_forward(const uint16_t *x, int64_t m, const nf4_weight &wt, const uint16_t *a,
                               const uint16_t *b, int32_t r, float s_lora, uint16_t *y,
                               uint16_t *t_ws, hipStream_t s) {
    const WView w = make_view(wt);
    const int64_t N = w.n, K = w.k;
    const int64_t rp = round64(r);  // adapter width padded to the K step (zeros)
    Params p{};
    p.lv = levels();
    p.splits = 1;
    if (r > 0) {
        // T'[m x rp] = s * X . A : Aop = X [m x K], Bop[c][k] = A[k][c] (columns of A)
        hipError_t e = lora_down<BF16_NN>(bf16_segment(x, K, K, a, r, K, r), m, rp, s_lora, t_ws, p.lv, s);
        if (e != hipSuccess) return e;
    }
    if (fwd_main_supported(K)) return launch_fwd_main(x, m, wt, r > 0 ? t_ws : nullptr, rp, b, r, y, s);
    p.seg[0] = nf4_segment(x, K, K, w);
    p.nseg = 1;
    if (r > 0) {
        // Y += T' . B : Aop = T' [m x rp], Bop[n][j] = B[j][n] (columns of B)
        p.seg[1] = bf16_segment(t_ws, rp, rp, b, N, r, N);
        p.nseg = 2;
    }
    p.M = m;
    p.Nc = N;
    p.c = y;
    p.ldc = N;
    p.out_scale = 1.0f;
    return run<256, 256, NF4_NT, BF16_NN>(p, s);
}

// Input gradient: U' = s dY.B^T (when r > 0), then dX = dY.W' + U'.A^T.
hipError_t launch_gemm_dgrad(const uint16_t *dy, int64_t m, const nf4_weight &wt, const uint16_t *a,
                             const uint16_t *b, int32_t r, float s_lora, uint16_t *dx,
                             uint16_t *u_ws, hipStream_t s) {
    const WView w = make_view(wt);
    const int64_t N = w.n, K = w.k;
    const int64_t rp = round64(r);
    Params p{};
    p.lv = levels();
    p.splits = 1;
    if (r > 0) {
        // U'[m x rp] = s * dY . B^T : Aop = dY [m x N], Bop[c][j] = B[c][j] (rows of B)
        hipError_t e = lora_down<BF16_NT>(bf16_segment(dy, N, N, b, N, r, N), m, rp, s_lora, u_ws, p.lv, s);
        if (e != hipSuccess) return e;
    }
    if (dgrad_main_supported(N, K)) return launch_dgrad_main(dy, m, wt, r > 0 ? u_ws : nullptr, rp, a, r, dx, s);
    p.seg[0] = nf4_segment(dy, N, N, w);
    p.nseg = 1;
    if (r > 0) {
        // dX += U' . A^T : Aop = U' [m x rp], Bop[c][j] = A[c][j] (rows of A)
        p.seg[1] = bf16_segment(u_ws, rp, rp, a, r, K, r);
        p.nseg = 2;
    }
    p.M = m;
    p.Nc = K;
    p.c = dx;
    p.ldc = K;
    p.out_scale = 1.0f;
    return run<256, 256, NF4_NN, BF16_NT>(p, s);
}

// Adapter gradients ([MF] "Gradient Computation"): T = X.A and U = dY.B^T
// (bf16, unscaled) by the down-projection, then two token sums (on the
// streaming kernel of linear_adapter.hip, or the generic kernel with a
// transposed A tile):
//   dA = s X^T U   [K x r]: Aop[k][i] = X[i][k], Bop[c][i] = U[i][c]
//   dB = s T^T dY  [r x N]: Aop[c][i] = T[i][c], Bop[n][i] = dY[i][n]
// Each token sum is split over up to kSplitMax workgroups per tile; its fp32
// partial sums are added, scaled by s and stored (bf16 or fp32) by one more
// pass. Workspace: T, U (lora_product_bytes of m rounded up to 64 each), then
// the partial sums. On the four-launch path T and U are stored transposed
// ([rp][lora_qt_row(m)]) for the token sums.
hipError_t launch_lora_grads(const uint16_t *x, const uint16_t *dy, int64_t m, int64_t K, int64_t N,
                             const uint16_t *a, const uint16_t *b, int32_t r, float s_lora, void *da, void *db,
                             bool f32_out, void *ws, hipStream_t s) {
    const int64_t rp = round64(r), mq = lora_qt_row(m);
    char *const base = static_cast<char *>(ws);
    uint16_t *const T = reinterpret_cast<uint16_t *>(base);
    uint16_t *const U = reinterpret_cast<uint16_t *>(base + lora_product_bytes(mq, rp));
    float *const part = reinterpret_cast<float *>(base + 2 * lora_product_bytes(mq, rp));
    const Levels lv = levels();
    hipError_t e = hipSuccess;
    const int64_t msteps = round64(m) / kBK;
    auto split_count = [](int64_t tiles, int64_t steps, int64_t target) {
        const int sp = (int)min((int64_t)kSplitMax, max((int64_t)1, (target + tiles - 1) / tiles));
        return (int)min((int64_t)sp, max((int64_t)1, steps));
    };
    if (m > 0 && da && db && adapter_down_supported(true, K, K, r, r) && adapter_down_supported(false, N, N, N, r) &&
        token_sum_supported(m, K, rp) && token_sum_supported(m, N, rp) && token_sum_qt_supported(m, rp)) {
        // Four launches: both down-projections (T = X.A, U = dY.B^T, fp32
        // partial sums even without a split), their split sums written
        // transposed (T^T, U^T [rp][mq]), both token sums (dA, dB), their
        // split sums.
        const int64_t mt = (m + 63) / 64, ct = rp / 64;
        const int sT = split_count(mt * ct, K / kBK, 256), sU = split_count(mt * ct, N / kBK, 256);
        float *const part_u = part + (int64_t)sT * m * rp;
        const DownJob jt{x, K, K, a, r, sT, part, T};
        const DownJob ju{dy, N, N, b, N, sU, part_u, U};
        e = launch_adapter_down_pair(jt, ju, m, r, rp, 1.0f, s);
        if (e != hipSuccess) return e;
        e = reduce_transpose_pair(TransposeJob{part, sT, m, rp, mq, r, T}, TransposeJob{part_u, sU, m, rp, mq, r, U},
                                  1.0f, s);
        if (e != hipSuccess) return e;
        const int sA = split_count((K / 64) * ct, msteps, 256), sB = split_count((N / 64) * ct, msteps, 256);
        float *const part_b = part + (int64_t)sA * K * r;
        const TokenSumJob ja{x, U, K, false, sA, sA > 1 ? part : nullptr, da};
        const TokenSumJob jb{dy, T, N, true, sB, sB > 1 ? part_b : nullptr, db};
        e = launch_token_sum_pair(ja, jb, m, rp, r, f32_out, s_lora, mq, s);
        if (e != hipSuccess) return e;
        return reduce_pair(f32_out, ReduceJob{part, sA, sA > 1 ? K * r : 0, da},
                           ReduceJob{part_b, sB, sB > 1 ? (int64_t)r * N : 0, db}, s_lora, s);
    }
    if (m > 0) {
        if (db) {
            e = lora_down<BF16_NN>(bf16_segment(x, K, K, a, r, K, r), m, rp, 1.0f, T, lv, s, part);
            if (e != hipSuccess) return e;
        }
        if (da) {
            e = lora_down<BF16_NT>(bf16_segment(dy, N, N, b, N, r, N), m, rp, 1.0f, U, lv, s, part);
            if (e != hipSuccess) return e;
        }
    }
    const int64_t mk = round64(m);  // token steps of 64 (tokens past m read as zero)
    // the streaming kernel of linear_adapter.hip: C[o][j] = sum_t P[t][o] Q[t][j]
    auto stream_sum = [&](const uint16_t *pm, int64_t O, const uint16_t *qm, bool transposed,
                          void *out) -> hipError_t {
        const int64_t tiles = (O / 64) * (rp / 64), steps = mk / kBK;
        int splits = (int)min((int64_t)kSplitMax, max((int64_t)1, (1024 + tiles - 1) / tiles));
        splits = (int)min((int64_t)splits, max((int64_t)1, steps));
        hipError_t e2 = launch_token_sum(pm, qm, m, O, rp, r, splits, splits > 1 ? part : nullptr, out, f32_out,
                                         transposed, s_lora, s);
        if (e2 != hipSuccess || splits == 1) return e2;
        const int64_t count = O * (int64_t)r;
        const dim3 grid((unsigned)((count / 4 + 255) / 256));
        if (f32_out)
            reduce_partials_kernel<true><<<grid, 256, 0, s>>>(part, splits, count, s_lora, out);
        else
            reduce_partials_kernel<false><<<grid, 256, 0, s>>>(part, splits, count, s_lora, out);
        return hipGetLastError();
    };
    // the generic kernel with a transposed A tile otherwise
    auto token_sum = [&](const uint16_t *at, int64_t lda, int64_t rows, const uint16_t *mat, int64_t ldm,
                         int64_t cols, void *out) -> hipError_t {
        Params q{};
        q.lv = lv;
        Segment sg{};
        sg.a = at;
        sg.lda = lda;
        sg.klen = mk;
        sg.a_krows = m;
        sg.mat = mat;
        sg.ldm = ldm;
        sg.mat_rows = m;
        sg.mat_cols = cols;
        q.seg[0] = sg;
        q.nseg = 1;
        q.M = rows;
        q.Nc = cols;
        q.ldc = cols;
        q.out_scale = s_lora;
        const int64_t tiles = ((rows + 63) / 64) * ((cols + 63) / 64), steps = mk / kBK;
        int splits = (int)min((int64_t)kSplitMax, max((int64_t)1, (512 + tiles - 1) / tiles));
        splits = (int)min((int64_t)splits, max((int64_t)1, steps));
        q.splits = splits;
        q.partial = part;
        hipError_t e2 = run<64, 64, BF16_NN, BF16_NN, true>(q, s);
        if (e2 != hipSuccess) return e2;
        const int64_t count = rows * cols;
        const dim3 grid((unsigned)((count / 4 + 255) / 256));
        if (f32_out)
            reduce_partials_kernel<true><<<grid, 256, 0, s>>>(part, splits, count, s_lora, out);
        else
            reduce_partials_kernel<false><<<grid, 256, 0, s>>>(part, splits, count, s_lora, out);
        return hipGetLastError();
    };
    if (da) {
        e = token_sum_supported(m, K, rp) ? stream_sum(x, K, U, false, da) : token_sum(x, K, K, U, rp, r, da);
        if (e != hipSuccess) return e;
    }
    if (db) e = token_sum_supported(m, N, rp) ? stream_sum(dy, N, T, true, db) : token_sum(T, rp, r, dy, N, N, db);
    return e;
}

}  // namespace nf4
