// linear_adapter.hip - the low-rank adapter's down-projection in the fused
// QLoRA linear for gfx950: the factor s (X A) of the forward ([MF] "Forward
// Pass Computation") and s (dY B^T) of the input gradient ([MF] "Gradient
// Computation"; source key in nf4_internal.h):
//   C[m x rp] = s * Aop[m x K] . Bop[rp x K]^T   (bf16 operands, fp32 sums)
// with Bop[c][k] = A[k][c] (forward, A [K x r]) or Bop[c][k] = B[c][k]
// (input gradient, B [r x N]); columns c >= r are zero.
//
// The product is thin (rp <= 256 columns) and long: it reads Aop (64 MiB at
// 4096 x 8192) once from HBM, so it is bound by that stream. A workgroup of
// 4 waves owns 64 rows x 64 columns and a slice of K (K is split over up to
// kSplitMax workgroups; the fp32 partial sums are added by a second pass).
// K advances 64 per step. Each step's Aop tile (64 rows x 128 B) goes global
// -> LDS by direct-to-LDS loads into a ring of kStages slots, issued
// kStages - 1 steps ahead; so does the Bop tile of the input gradient (rows
// of B). The forward's Bop operand is a column slice of A: each thread loads
// two 16-byte row pieces and stores them as they are into a row-major [k][c]
// tile a step before use, and the operand comes from the transposing LDS read
// (lds_read_tr16). The DMA-fed tiles are stored [row][64] with 16-byte chunks
// XOR-swizzled by row. The four waves split the 64 x 64 output 2 x 2 and run
// v_mfma_f32_16x16x32_bf16.
#include <type_traits>

#include "gemm_common.h"

namespace nf4 {
namespace {

using gemm::f32x4_t;
using gemm::lds_void;
using gemm::Rsrc;
using gemm::rsrc;
using gemm::vmcnt_at_most;
using gemm::lds_read_tr16;
using gemm::u32x2;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kBM = 64;                 // Aop rows per workgroup
constexpr int kBC = 64;                 // output columns per workgroup
constexpr int kBK = 64;                 // K step
constexpr int kStages = 4;              // LDS ring slots
constexpr int kTile = kBM * kBK * 2;    // one tile: 64 rows x 128 B
constexpr int kLoads = 4;               // vector-memory instructions per wave per step
static_assert(kBC == kBM, "Aop and Bop tiles share one layout");

// 16-byte chunk swizzle of a row-major 64 x 128 B tile read by the
// transposing LDS read (lds_read_tr16, gemm_common.h): chunk c of
// row r sits at c ^ tsig(r). The 8 rows that one half-wave's transposing
// reads touch (tau + q and tau + 16 + q, q < 4, tau % 8 in {0, 4}) then fall
// on 8 distinct 32-byte bank windows, and each 16-byte store instruction
// (8 consecutive rows, whole rows) fills the 64 banks 4 times over.
__device__ __forceinline__ int tsig(int r) { return 2 * ((r >> 1) & 1) + 4 * ((r >> 4) & 1); }

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`.
__device__ __forceinline__ uint32_t swz(int row, int chunk) {
    return (uint32_t)row * 128u + 16u * (uint32_t)(chunk ^ ((row >> 1) & 7));
}

struct AdapterParams {
    const uint16_t *a;   // Aop, row-major [m x lda]
    int64_t lda;
    const uint16_t *mat; // A [K x r] (forward) or B [r x ldm] (input gradient)
    int64_t ldm;
    int64_t m, klen, rp;
    int32_t r;
    int splits;
    float *partial;      // [splits][m][rp] fp32 sums, or nullptr
    uint16_t *c;         // [m][rp] bf16 = scale * sum when partial == nullptr
    float scale;
};

// kMode 0: Bop is B (input gradient), 1: Bop is A^T (forward), 2: both in one
// launch, products p0 (forward form) for blockIdx.z < p0.rp / 64 and p1
// (input-gradient form) above.
template <int kMode>
__global__ __launch_bounds__(kThreads) void adapter_down_kernel(AdapterParams p0, AdapterParams p1) {
    // One static object per ring slot, so that the compiler's waits for a
    // direct-to-LDS load cover only reads of its own slot.
    __shared__ __align__(16) char s_x0[kTile], s_x1[kTile], s_x2[kTile], s_x3[kTile];
    __shared__ __align__(16) char s_b0[kTile], s_b1[kTile], s_b2[kTile], s_b3[kTile];
    auto xs = [&](auto SC) -> char * {
        constexpr int s = decltype(SC)::value;
        if constexpr (s == 0) return s_x0;
        else if constexpr (s == 1) return s_x1;
        else if constexpr (s == 2) return s_x2;
        else return s_x3;
    };
    auto bs = [&](auto SC) -> char * {
        constexpr int s = decltype(SC)::value;
        if constexpr (s == 0) return s_b0;
        else if constexpr (s == 1) return s_b1;
        else if constexpr (s == 2) return s_b2;
        else return s_b3;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    auto body = [&](const AdapterParams &p, auto NNC, const int cg) {  // cg: 64-column group of C
        constexpr bool kNN = decltype(NNC)::value;
        if ((int)blockIdx.y >= p.splits) return;  // (a paired launch sizes y for the larger split)
        const int t = threadIdx.x, lane = t & 63;
        const int w = __builtin_amdgcn_readfirstlane(t >> 6);
        const int lr = lane & 15, g = lane >> 4;
        const int64_t m0 = (int64_t)blockIdx.x * kBM;
        const int64_t steps = p.klen / kBK;
        const int64_t per = (steps + p.splits - 1) / p.splits;
        const int64_t s_lo = min(steps, (int64_t)blockIdx.y * per);
        const int n = (int)(min(steps, s_lo + per) - s_lo);
        const int64_t m_rows = min((int64_t)kBM, p.m - m0);
        const Rsrc none = rsrc(p.a, 0);

        // Aop tile: wave w moves rows 16w .. 16w+15, 8 rows per load; lane l of
        // load q fills row 16w + 8q + l/8, physical chunk l % 8, which holds
        // logical chunk (l % 8) ^ ((row >> 1) & 7). Rows past m read as zeros
        // (the row is in the range-checked lane offset, K in the scalar offset).
        const Rsrc x_rs = rsrc(p.a + m0 * p.lda, m_rows * p.lda * 2);
        uint32_t x_off[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = 16 * w + 8 * q + (lane >> 3);
            x_off[q] = (uint32_t)(row * p.lda * 2 + ((lane & 7) ^ ((row >> 1) & 7)) * 16);
        }

        // Bop tile, input gradient: rows c of B, moved like the Aop tile.
        const int64_t c_rows = max((int64_t)0, min((int64_t)kBC, (int64_t)p.r - (int64_t)cg * kBC));
        const Rsrc bt_rs = rsrc(p.mat + (int64_t)cg * kBC * p.ldm, kNN ? 0 : c_rows * p.ldm * 2);
        uint32_t bt_off[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int row = 16 * w + 8 * q + (lane >> 3);
            bt_off[q] = (uint32_t)(row * p.ldm * 2 + ((lane & 7) ^ ((row >> 1) & 7)) * 16);
        }

        // Bop tile, forward: thread (kp = 8w + lane / 8, cc = lane % 8) loads A
        // rows 2kp and 2kp + 1 of the step, columns 64 cg + 8cc .. + 7 (all
        // valid or all past r, as r % 8 == 0); each octet of lanes reads one
        // row's 128 contiguous bytes. A column chunk past r takes the lane offset
        // num_records, out of range with or without the scalar offset (the
        // descriptor stays wave-uniform).
        const int kp = 8 * w + (lane >> 3), cc = lane & 7;
        const bool cc_live = (int64_t)cg * kBC + 8 * cc < p.r;
        const int64_t bn_bytes = kNN ? p.klen * p.ldm * 2 : 0;
        const Rsrc bn_rs = rsrc(p.mat, bn_bytes);
        // forward: the step's 64 rows of A (columns 64 cg .. +63) go to LDS
        // row-major, [k][c] with the tsig swizzle: thread (w, lane), load h:
        // row 16 w + 8 h + lane / 8, columns 8 (lane % 8) .. +7 (past r the
        // lane offset is pushed out of the descriptor's range)
        uint32_t bn_o[2], bn_lds[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int row = 16 * w + 8 * h2 + (lane >> 3);
            bn_o[h2] = cc_live ? (uint32_t)((row * p.ldm + (int64_t)cg * kBC + 8 * cc) * 2) : (uint32_t)bn_bytes;
            bn_lds[h2] = (uint32_t)(row * 128 + 16 * (cc ^ tsig(row)));
        }
        u32x4 braw[kStages][2];

        // Loads of this workgroup's step i into ring slot SC (i % kStages): always
        // issued, through the empty descriptor for steps past the slice.
        auto issue = [&](int i, auto SC) {
            const bool live = i < n;
            const int64_t k0 = (s_lo + (live ? i : 0)) * kBK;
            // (scalar offsets: uniform by construction, said so for the compiler)
            const int so_k = __builtin_amdgcn_readfirstlane((int)(k0 * 2));
            const Rsrc xr = live ? x_rs : none;
            char *xd = xs(SC) + 16 * w * 128;
#pragma unroll
            for (int q = 0; q < 2; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void *)(xd + q * 1024), 16, x_off[q], so_k, 0,
                                                         0);
            if constexpr (!kNN) {
                const Rsrc br = live ? bt_rs : none;
                char *bd = bs(SC) + 16 * w * 128;
#pragma unroll
                for (int q = 0; q < 2; ++q)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void *)(bd + q * 1024), 16, bt_off[q], so_k,
                                                             0, 0);
            } else {
                constexpr int s = decltype(SC)::value;
                const Rsrc br = live ? bn_rs : none;
                const int so = __builtin_amdgcn_readfirstlane((int)(k0 * p.ldm * 2));
                braw[s][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(br, bn_o[0], so, 0));
                braw[s][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(br, bn_o[1], so, 0));
            }
        };
        // Forward: the rows of A of the step in slot SC, stored as loaded.
        auto write_bn = [&](auto SC) {
            if constexpr (kNN) {
                constexpr int s = decltype(SC)::value;
                char *bd = bs(SC);
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) *reinterpret_cast<u32x4 *>(bd + bn_lds[h2]) = braw[s][h2];
            }
        };

        // MFMA fragments: wave (wr, wc) owns rows 32 wr .. +31, columns 32 wc .. +31;
        // tile row 16i + lr, logical chunk 2g + ks.
        const int wr = w >> 1, wc = w & 1;
        uint32_t fa[2][2], fb[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                fa[i][ks] = swz(32 * wr + 16 * i + lr, 2 * g + ks);
                fb[i][ks] = swz(32 * wc + 16 * i + lr, 2 * g + ks);
            }
        // forward: Bop of column tile i, substep ks by two transposing reads
        // h2 of the row-major A tile: lane (lr, g) points at row
        // 16 g + 8 ks + 4 h2 + lr / 4, columns 32 wc + 16 i + 4 (lr % 4) .. +3,
        // and receives rows (k) 16 g + 8 ks + 4 h2 .. +3 of column
        // 32 wc + 16 i + lr, the k order of the Aop fragments
        uint32_t trb[2][2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int tau = 16 * g + 8 * ks + 4 * h2 + (lr >> 2);
                    const int c = 4 * wc + 2 * i + ((lr & 3) >> 1);
                    trb[i][ks][h2] = (uint32_t)(tau * 128 + 16 * (c ^ tsig(tau)) + 8 * (lr & 1));
                }
        f32x4_t acc[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // Step i from slot SC; the loads of step i + kStages - 1 go to slot SI.
        auto step = [&](int i, auto SC, auto SN, auto SI) {
            // This wave's loads of step i have landed once at most the loads of
            // the two later steps are outstanding; LDS writes are done too. The
            // barrier then makes every wave's part of the tiles visible, and all
            // waves have finished step i - 1, so its slot can be refilled.
            __builtin_amdgcn_s_waitcnt(vmcnt_at_most((kStages - 2) * kLoads) & ~(0xF << 8));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            issue(i + kStages - 1, SI);
            write_bn(SN);  // forward: Bop tile of step i + 1
            if (i < n) {
                const char *xa = xs(SC), *xb = bs(SC);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    u32x4 a[2], b[2];
#pragma unroll
                    for (int i2 = 0; i2 < 2; ++i2) {
                        a[i2] = *reinterpret_cast<const u32x4 *>(xa + fa[i2][ks]);
                        if constexpr (kNN) {
                            const u32x2 lo = lds_read_tr16(xb + trb[i2][ks][0]);
                            const u32x2 hi = lds_read_tr16(xb + trb[i2][ks][1]);
                            b[i2] = u32x4{lo.x, lo.y, hi.x, hi.y};
                        } else {
                            b[i2] = *reinterpret_cast<const u32x4 *>(xb + fb[i2][ks]);
                        }
                    }
#pragma unroll
                    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i2][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, a[i2]), __builtin_bit_cast(bf16x8_t, b[j]),
                                acc[i2][j], 0, 0, 0);
                }
            }
        };

        issue(0, S0{});
        issue(1, S1{});
        issue(2, S2{});
        write_bn(S0{});
        for (int i = 0; i < n; i += kStages) {
            step(i, S0{}, S1{}, S3{});
            step(i + 1, S1{}, S2{}, S0{});
            step(i + 2, S2{}, S3{}, S1{});
            step(i + 3, S3{}, S0{}, S2{});
        }
        // no direct-to-LDS load may still be in flight when the workgroup ends
        __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));

        // D row 4g + q, column lr of each 16 x 16 tile; columns from r to rp are
        // written as zeros whatever the padding rows of the tiles held.
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t col = (int64_t)cg * kBC + 32 * wc + 16 * j + lr;
                const bool col_live = col < p.r;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t row = m0 + 32 * wr + 16 * i + 4 * g + q;
                    if (row >= p.m) continue;
                    const float v = col_live ? acc[i][j][q] : 0.0f;
                    if (p.partial)
                        p.partial[((int64_t)blockIdx.y * p.m + row) * p.rp + col] = v;
                    else
                        p.c[row * p.rp + col] = (uint16_t)(pack_bf16x2(v * p.scale, 0.0f) & 0xFFFFu);
                }
            }

    };
    if constexpr (kMode == 2) {
        const int z_nn = (int)(p0.rp / kBC);
        if ((int)blockIdx.z < z_nn)
            body(p0, std::true_type{}, (int)blockIdx.z);
        else
            body(p1, std::false_type{}, (int)blockIdx.z - z_nn);
    } else {
        body(p0, std::integral_constant<bool, kMode == 1>{}, (int)blockIdx.z);
    }
}

// ---- token sums of the adapter gradients ([MF] "Gradient Computation"):
//   C[o][j] = sum over tokens t of P[t][o] * Q[t][j]
// with P = X, Q = dY.B^T (dA = s X^T (dY B^T), C = dA, [O x r]) or P = dY,
// Q = X.A (dB = s (X A)^T dY, C^T = dB, [r x O]). Both operands have the
// tokens as rows, so both are transposed on the way into LDS: each thread
// loads two token rows of 8 columns of P and of Q and writes their 8 column
// pairs. A workgroup of 4 waves owns 64 x 64 of C and a slice of the tokens;
// loads run 3 steps of 64 tokens ahead through a register ring, and the LDS
// tiles of a step are written one step before use.
// With kQT, Q arrives transposed (Q^T [rp x qs], tokens contiguous, zeros
// past m), written so by the split-sum pass of the down-projections. Its tile
// rows are then already [column][token] runs of 128 bytes: each thread loads
// two 16-byte chunks (through the same register ring) and stores them as they
// are. P is not turned around in registers either: its tile stays row-major
// ([token][column], 16-byte stores) and the MFMA operand comes from gfx950's
// transposing LDS read, ds_read_b64_tr_b16 (lds_read_tr16). Within each group
// of 16 lanes that read returns to lane i the 16-bit element i % 4 of the
// 8-byte pieces addressed by lanes i / 4, i / 4 + 4, i / 4 + 8, i / 4 + 12;
// with lane j pointing at token row tau + j / 4, columns 4 (j % 4) .. +3 of
// an operand's 16 columns, lane i receives tokens tau .. tau + 3 of column i.
// Two such reads make the lane's 8 tokens. No permutes are left in the step.

struct TokenSumParams {
    const uint16_t *p;  // [m x O] row-major
    const uint16_t *q;  // [m x rp] row-major
    int64_t m, O, rp;
    int32_t r;
    int splits;
    float *partial;     // [splits][O][r] (or [splits][r][O] when transposed), or nullptr
    void *out;          // final C (splits == 1): fp32 or bf16, [O x r] or [r x O]
    bool f32, transposed;
    float scale;
    int64_t qs;         // with Q transposed: the row length of Q^T in tokens
};

// Workgroups with blockIdx.x < x1 run the sums of p0, the others those of p1
// (blockIdx.x - x1); one launch then covers both adapter gradients.
template <bool kQT>
__global__ __launch_bounds__(kThreads) void token_sum_kernel(TokenSumParams p0, TokenSumParams p1, int x1) {
    __shared__ __align__(16) char s_p0[kTile], s_p1[kTile], s_q0[kTile], s_q1[kTile];
    auto ps = [&](auto SC) -> char * {
        if constexpr (decltype(SC)::value == 0) return s_p0;
        else return s_p1;
    };
    auto qs = [&](auto SC) -> char * {
        if constexpr (decltype(SC)::value == 0) return s_q0;
        else return s_q1;
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;

    // The body runs from two uniform branches, one per job, so the compiler
    // never selects between the two parameter blocks at run time (a select
    // of the whole struct went through scratch memory).
    auto body = [&](const TokenSumParams &p, const int bx) {
    if ((int)blockIdx.y >= p.splits) return;  // (sized for the larger split of the two)
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lr = lane & 15, g = lane >> 4;
    const int64_t o0 = (int64_t)bx * kBM;
    const int cg = blockIdx.z;
    const int64_t steps = (p.m + kBK - 1) / kBK;
    const int64_t per = (steps + p.splits - 1) / p.splits;
    const int64_t s_lo = min(steps, (int64_t)blockIdx.y * per);
    const int n = (int)(min(steps, s_lo + per) - s_lo);
    const Rsrc none = rsrc(p.p, 0);

    // thread (kp, cc): token rows 2kp and 2kp + 1 of the step, columns
    // 8cc .. 8cc + 7 of the tile (of P: o0 + 8cc; of Q: 64 cg + 8cc, which
    // are all valid or all past r as r % 8 == 0: past r the lane offset is
    // pushed out of the descriptor's range). Each octet of lanes reads one
    // row's 128 contiguous bytes, so a load instruction covers 8 rows x 128 B.
    const int kp = 8 * w + (lane >> 3), cc = lane & 7;
    const bool q_live = (int64_t)cg * kBC + 8 * cc < p.r;
    const uint32_t p_off = (uint32_t)((2 * kp * p.O + o0 + 8 * cc) * 2);
    const uint32_t q_off = q_live ? (uint32_t)((2 * kp * p.rp + (int64_t)cg * kBC + 8 * cc) * 2) : 0xFFFFFFF0u;
    u32x4 raw[4][4];  // [ring slot][P row 0, P row 1, Q row 0, Q row 1] (kQT: Q^T chunks 0, 1)
    // kQT: thread (w, lane), chunk h: tile row 16w + 8h + lane/8, tokens
    // 8 (lane % 8) .. +7 of the step
    uint32_t qt_off[2], qt_lds[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 16 * w + 8 * h + (lane >> 3);
        qt_off[h] = kQT ? (uint32_t)((((int64_t)cg * kBC + row) * p.qs + 8 * (lane & 7)) * 2) : 0u;
        qt_lds[h] = swz(row, lane & 7);
    }
    // kQT: the P tile row-major. Thread (w, lane), load h: token row
    // 16w + 8h + lane/8, columns o0 + 8 (lane % 8) .. +7 (each load
    // instruction 8 rows x 128 contiguous bytes), stored at chunk
    // (lane % 8) ^ tsig(row).
    uint32_t pt_off[2], pt_lds[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 16 * w + 8 * h + (lane >> 3);
        pt_off[h] = kQT ? (uint32_t)((row * p.O + o0 + 8 * (lane & 7)) * 2) : 0u;
        pt_lds[h] = (uint32_t)(row * 128 + 16 * ((lane & 7) ^ tsig(row)));
    }

    // Loads of step i (ring slot SC): descriptors start at the step's first
    // token and end at token m, so tokens past m read as zeros.
    auto issue = [&](int i, auto SC) {
        constexpr int sl = decltype(SC)::value;
        const bool live = i < n;
        const int64_t tok0 = (s_lo + (live ? i : 0)) * kBK;
        const int64_t rows = live ? min((int64_t)kBK, p.m - tok0) : 0;
        const Rsrc pr = live ? rsrc(p.p + tok0 * p.O, rows * p.O * 2) : none;
        raw[sl][0] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, kQT ? pt_off[0] : p_off, 0, 0));
        raw[sl][1] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, kQT ? pt_off[1] : p_off + (uint32_t)(p.O * 2), 0, 0));
        if constexpr (kQT) {
            // the Q^T tile: chunk h is tokens 8 (lane % 8) .. +7 of tile row
            // (column) 16 w + 8 h + lane / 8. The descriptor starts at the
            // step's first token; Q^T rows hold whole steps, so every access
            // stays inside Q^T.
            const Rsrc qr = live ? rsrc(p.q + tok0, (p.rp * p.qs - tok0) * 2) : none;
            raw[sl][2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, qt_off[0], 0, 0));
            raw[sl][3] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, qt_off[1], 0, 0));
        } else {
            const Rsrc qr = live ? rsrc(p.q + tok0 * p.rp, rows * p.rp * 2) : none;
            raw[sl][2] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, q_off, 0, 0));
            raw[sl][3] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, q_live ? q_off + (uint32_t)(p.rp * 2) : q_off, 0, 0));
        }
    };

    // The column pairs of ring slot SR to LDS slot SL ([column][token] tiles).
    auto write = [&](auto SR, auto SL) {
        constexpr int sl = decltype(SR)::value;
        char *pd = ps(SL), *qd = qs(SL);
        if constexpr (kQT) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                *reinterpret_cast<u32x4 *>(pd + pt_lds[h]) = raw[sl][h];
                *reinterpret_cast<u32x4 *>(qd + qt_lds[h]) = raw[sl][2 + h];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                const uint32_t off = swz(8 * cc + j, kp >> 2) + 4 * (kp & 3);
                const uint32_t a0 = raw[sl][0][j >> 1], a1 = raw[sl][1][j >> 1];
                const uint32_t b0 = raw[sl][2][j >> 1], b1 = raw[sl][3][j >> 1];
                *reinterpret_cast<uint32_t *>(pd + off) = __builtin_amdgcn_perm(a1, a0, sel);
                *reinterpret_cast<uint32_t *>(qd + off) = __builtin_amdgcn_perm(b1, b0, sel);
            }
        }
    };

    const int wr = w >> 1, wc = w & 1;
    uint32_t fa[2][2], fb[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            fa[i][ks] = swz(32 * wr + 16 * i + lr, 2 * g + ks);
            fb[i][ks] = swz(32 * wc + 16 * i + lr, 2 * g + ks);
        }
    // kQT: the two transposing reads h of the P operand of row tile i and
    // substep ks: lane (lr, g) points at token row tau = 16g + 8ks + 4h + lr/4,
    // columns 32wr + 16i + 4 (lr % 4) .. +3 (logical chunk 4wr + 2i +
    // (lr % 4) / 2, byte 8 (lr % 2) within it), and receives tokens
    // 16g + 8ks + 4h .. +3 of column 32wr + 16i + lr.
    uint32_t tr_off[2][2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tau = 16 * g + 8 * ks + 4 * h + (lr >> 2);
                const int c = 4 * wr + 2 * i + ((lr & 3) >> 1);
                tr_off[i][ks][h] = (uint32_t)(tau * 128 + 16 * (c ^ tsig(tau)) + 8 * (lr & 1));
            }
    f32x4_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Step i: the tiles of step i are in LDS slot i & 1 (written last step);
    // issue the loads of step i + 3 into ring slot SI, write step i + 1's
    // tiles (ring slot SN) to the other LDS slot, then the MFMAs.
    auto step = [&](int i, auto SC, auto SN, auto SI, auto LC, auto LN) {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's tile writes are done
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(i + 3, SI);
        write(SN, LN);
        if (i < n) {
            const char *xa = ps(LC), *xb = qs(LC);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                u32x4 a[2], b[2];
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2) {
                    if constexpr (kQT) {
                        const gemm::u32x2 lo = gemm::lds_read_tr16(xa + tr_off[i2][ks][0]);
                        const gemm::u32x2 hi = gemm::lds_read_tr16(xa + tr_off[i2][ks][1]);
                        a[i2] = u32x4{lo.x, lo.y, hi.x, hi.y};
                    } else {
                        a[i2] = *reinterpret_cast<const u32x4 *>(xa + fa[i2][ks]);
                    }
                    b[i2] = *reinterpret_cast<const u32x4 *>(xb + fb[i2][ks]);
                }
#pragma unroll
                for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i2][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, a[i2]), __builtin_bit_cast(bf16x8_t, b[j]),
                            acc[i2][j], 0, 0, 0);
            }
        }
        (void)SC;
    };

    issue(0, S0{});
    issue(1, S1{});
    issue(2, S2{});
    write(S0{}, S0{});
    for (int i = 0; i < n; i += 4) {
        step(i, S0{}, S1{}, S3{}, S0{}, S1{});
        step(i + 1, S1{}, S2{}, S0{}, S1{}, S0{});
        step(i + 2, S2{}, S3{}, S1{}, S0{}, S1{});
        step(i + 3, S3{}, S0{}, S2{}, S1{}, S0{});
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_at_most(0));  // the loads of steps past the slice

    // D row 4g + q (o), column lr (j) of each 16 x 16 tile; columns past r
    // are not stored
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int64_t j = (int64_t)cg * kBC + 32 * wc + 16 * jt + lr;
            const int64_t o = o0 + 32 * wr + 16 * i + 4 * g;
            if (j >= p.r) continue;
            const f32x4_t v = acc[i][jt];
            if (p.partial) {
                float *dst = p.partial + (int64_t)blockIdx.y * p.O * p.r;
                if (p.transposed) {
                    *reinterpret_cast<f32x4_t *>(dst + j * p.O + o) = v;
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) dst[(o + q) * p.r + j] = v[q];
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t idx = p.transposed ? j * p.O + o + q : (o + q) * p.r + j;
                    const float x = v[q] * p.scale;
                    if (p.f32) static_cast<float *>(p.out)[idx] = x;
                    else static_cast<uint16_t *>(p.out)[idx] = (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFFu);
                }
            }
        }
    };
    if ((int)blockIdx.x >= x1)
        body(p1, (int)blockIdx.x - x1);
    else
        body(p0, (int)blockIdx.x);
}

}  // namespace

bool token_sum_supported(int64_t m, int64_t O, int64_t rp) {
    // 32-bit buffer offsets within one step's 64 token rows
    return O % kBM == 0 && 64 * O * 2 < ((int64_t)1 << 31) && 64 * rp * 2 < ((int64_t)1 << 31) && m >= 0;
}

namespace {
TokenSumParams token_params(const uint16_t *pm, const uint16_t *qm, int64_t m, int64_t O, int64_t rp, int32_t r,
                            int splits, float *partial, void *out, bool f32, bool transposed, float scale,
                            int64_t qs = 0) {
    TokenSumParams p{};
    p.p = pm;
    p.q = qm;
    p.m = m;
    p.O = O;
    p.rp = rp;
    p.r = r;
    p.splits = max(1, splits);
    p.partial = partial;
    p.out = out;
    p.f32 = f32;
    p.transposed = transposed;
    p.scale = scale;
    p.qs = qs;
    return p;
}
}  // namespace

hipError_t launch_token_sum(const uint16_t *pm, const uint16_t *qm, int64_t m, int64_t O, int64_t rp, int32_t r,
                            int splits, float *partial, void *out, bool f32, bool transposed, float scale,
                            hipStream_t s) {
    const TokenSumParams p = token_params(pm, qm, m, O, rp, r, splits, partial, out, f32, transposed, scale);
    const dim3 grid((unsigned)(O / kBM), (unsigned)p.splits, (unsigned)(rp / kBC));
    token_sum_kernel<false><<<grid, kThreads, 0, s>>>(p, p, (int)grid.x);
    return hipGetLastError();
}

hipError_t launch_token_sum_pair(const TokenSumJob &a, const TokenSumJob &b, int64_t m, int64_t rp, int32_t r,
                                 bool f32, float scale, int64_t qt, hipStream_t s) {
    const TokenSumParams pa = token_params(a.pm, a.qm, m, a.O, rp, r, a.splits, a.partial, a.out, f32,
                                           a.transposed, scale, qt);
    const TokenSumParams pb = token_params(b.pm, b.qm, m, b.O, rp, r, b.splits, b.partial, b.out, f32,
                                           b.transposed, scale, qt);
    const int xa = (int)(a.O / kBM);
    const dim3 grid((unsigned)(xa + b.O / kBM), (unsigned)max(pa.splits, pb.splits), (unsigned)(rp / kBC));
    if (qt > 0)
        token_sum_kernel<true><<<grid, kThreads, 0, s>>>(pa, pb, xa);
    else
        token_sum_kernel<false><<<grid, kThreads, 0, s>>>(pa, pb, xa);
    return hipGetLastError();
}

bool adapter_down_supported(bool nn, int64_t lda, int64_t klen, int64_t ldm, int32_t r) {
    // 32-bit buffer offsets: a tile's 64 rows of Aop (or of B), and all of A
    if (lda > ((int64_t)1 << 23) || klen % kBK != 0) return false;
    if (nn) return klen * ldm * 2 < ((int64_t)1 << 31);
    return ldm <= ((int64_t)1 << 23) && (int64_t)r * ldm * 2 < ((int64_t)1 << 31);
}

namespace {
AdapterParams down_params(const uint16_t *aop, int64_t lda, int64_t m, int64_t klen, const uint16_t *mat,
                          int64_t ldm, int32_t r, int64_t rp, int splits, float *partial, uint16_t *c, float scale) {
    AdapterParams p{};
    p.a = aop;
    p.lda = lda;
    p.mat = mat;
    p.ldm = ldm;
    p.m = m;
    p.klen = klen;
    p.rp = rp;
    p.r = r;
    p.splits = max(1, splits);
    p.partial = partial;
    p.c = c;
    p.scale = scale;
    return p;
}
}  // namespace

hipError_t launch_adapter_down(bool nn, const uint16_t *aop, int64_t lda, int64_t m, int64_t klen,
                               const uint16_t *mat, int64_t ldm, int32_t r, int64_t rp, int splits,
                               float *partial, uint16_t *c, float scale, hipStream_t s) {
    const AdapterParams p = down_params(aop, lda, m, klen, mat, ldm, r, rp, splits, partial, c, scale);
    const dim3 grid((unsigned)((m + kBM - 1) / kBM), (unsigned)p.splits, (unsigned)(rp / kBC));
    if (nn)
        adapter_down_kernel<1><<<grid, kThreads, 0, s>>>(p, p);
    else
        adapter_down_kernel<0><<<grid, kThreads, 0, s>>>(p, p);
    return hipGetLastError();
}

hipError_t launch_adapter_down_pair(const DownJob &fwd, const DownJob &bwd, int64_t m, int32_t r, int64_t rp,
                                    float scale, hipStream_t s) {
    const AdapterParams pa = down_params(fwd.aop, fwd.lda, m, fwd.klen, fwd.mat, fwd.ldm, r, rp, fwd.splits,
                                         fwd.partial, fwd.c, scale);
    const AdapterParams pb = down_params(bwd.aop, bwd.lda, m, bwd.klen, bwd.mat, bwd.ldm, r, rp, bwd.splits,
                                         bwd.partial, bwd.c, scale);
    const dim3 grid((unsigned)((m + kBM - 1) / kBM), (unsigned)max(pa.splits, pb.splits), (unsigned)(2 * rp / kBC));
    adapter_down_kernel<2><<<grid, kThreads, 0, s>>>(pa, pb);
    return hipGetLastError();
}

}  // namespace nf4
