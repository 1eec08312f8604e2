// linear_fwd.hip - large-M fused NF4 linear forward for gfx950 on bf16 MFMA
// ([MF] "Forward Pass Computation"; source key in nf4_internal.h):
//   Y = X . W'^T + T' . B,   T' = s (X . A) (bf16, computed beforehand),
// W' = dequantize(W), W stored [N x K] NF4 (64-blocks along K).
//
// Tile: a workgroup of 4 waves owns 256 rows x 256 columns of Y; wave w owns
// all 256 rows of columns 64w .. 64w+63, as 8 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, in AGPRs). K
// advances 64 (one NF4 block) per step, in 4 substeps of 16.
//
// Why the 32 x 32 form: one wave per SIMD issues the MFMAs and all the work
// around them (fragment reads, level-table reads, dequantization, loads).
// Measured on gfx950, a 16x16x32 MFMA (16 cycles) hides about 2 other
// instructions and each further one costs its issue time, while a 32x32x16
// MFMA (32 cycles) hides about 6: per flop, the dequantization of the W
// operand fits in the matrix cores' shadow.
//
// K order: the MFMA contracts 16 k per substep, 8 from each lane half. Within
// a step the 64 k are ordered so that lane half h (lanes 32h .. 32h+31) covers
// k = 32h .. 32h+31 (substep ks: 32h + 8ks .. +7), for X and W alike, so a
// lane's W codes for a step are one 16-byte load: 32 codes of one weight row.
//
//  - X goes global -> LDS directly (buffer_load ... lds, no registers), three
//    tiles in flight, in the tile_seg layout (gemm_common.h): conflict-free
//    fragment reads.
//  - W never touches LDS: each lane dequantizes its codes in registers through
//    a 256-entry (low, high) level table in LDS, the levels held as fp16 (see
//    level_pair), and one v_fma_mix_f32 per weight (exact fp16 widening x c1'
//    in fp32), packed to bf16.
//  - The W operands of substep ks+1 are built during substep ks: their level
//    reads in its first 8 MFMA slots, their arithmetic in the last 8.
// All loads are raw buffer loads with per-tile descriptors whose size stops
// at the last valid row: rows beyond M or N read as zero, the loop has no
// branches, and the per-step advance is a scalar offset.
#include <utility>

#include "gemm_common.h"

namespace nf4 {
namespace {

using namespace gemm;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kTM = kBM / 32;                // 8 row tiles per wave
constexpr int kTN = 64 / 32;                 // 2 column tiles per wave
constexpr int kATile = kBM * kBK * 2;        // 32 KiB of bf16 per X tile
constexpr int kTable = 256 * 256;            // level-pair table, one copy per lane
constexpr int kPairs = 4 * kTM;              // X fragments (MFMA pairs) per step
constexpr int kFragAhead = 6;                // fragments read this many pairs ahead
constexpr int kFragRing = 8;
constexpr int kUnits = 4 * kTN;              // level pairs per substep's W operands
// the first slot that reads the next step's X tile
constexpr int kBarrierSlot = 2 * (kPairs - kFragAhead);
static_assert(kPairs % kFragRing == 0 && kFragRing > kFragAhead, "fragment ring keeps its phase");
// all of a step's loads are issued before its barrier: X tile part q at slot
// 6q + 3, the codes of column tile j at slot 12j + 1
static_assert(6 * 7 + 3 < kBarrierSlot && 12 * (kTN - 1) + 1 < kBarrierSlot, "loads before the barrier");
static_assert(kUnits == 8, "one level read per slot in the first half of a substep");

struct FwdParams {
    const uint16_t *x;      // X [M x K]
    int64_t M, K, N;
    const uint8_t *codes;   // W codes [N x K/2]
    const uint8_t *q8;      // E4M3 codes of c1/c2 (double quantization) or nullptr
    const float *c2;
    int64_t n_groups;       // entries of c2
    const float *absmax;    // c1 (no double quantization)
    const uint16_t *t;      // T' [M x rp] bf16, or nullptr (no adapter)
    int64_t rp;             // adapter width padded to 64
    const uint16_t *b;      // B [r x N] bf16
    int32_t r;
    uint16_t *y;            // Y [M x N] bf16
    Levels lv;
};

__device__ __forceinline__ void mfma32(f32x16_t &c, const u32x4 &a, const u32x4 &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

// Level-pair table in LDS: the entry of code byte b holds (q[b & 15],
// q[b >> 4]) as two fp16 (a 4-byte entry, half the LDS bytes of an fp32
// pair). Each lane has its own copy, entry b of lane l at byte 256 b + 4 l,
// so the lanes of a wave read distinct banks whatever the code bytes. For
// byte h of the code dword d, v_perm builds the address (b << 8) | 4 l in one
// instruction. The fp16 levels differ from the fp32 ones by at most 2^-12
// relative, far below the bf16 rounding of the operand.
// The table is a static LDS array: its base folds into the read's offset.
__device__ __forceinline__ uint32_t level_pair(const char *tab, uint32_t d, int h, uint32_t lane4) {
    const uint32_t addr = __builtin_amdgcn_perm(d, lane4, 0x0C0C0400u | ((uint32_t)h << 8));
    return *reinterpret_cast<const uint32_t *>(tab + addr);
}

// Codes and scale inputs of one K-step for a lane's column tiles.
struct Raw {
    u32x4 c[kTN];     // 32 codes: k = 32h .. 32h+31 of the block
    uint32_t q[kTN];  // E4M3 code of c1/c2 (double quantization)
    float s[kTN];     // c2 (double quantization) or c1
};

template <bool kDQ>
__global__ __launch_bounds__(kThreads) void gemm_fwd_kernel(FwdParams p) {
    // Static LDS: the table and three X tiles as separate objects, so that the
    // compiler's waits for a direct-to-LDS load cover only reads of its tile.
    __shared__ __align__(16) char s_tab[kTable];
    __shared__ __align__(16) char s_x0[kATile];
    __shared__ __align__(16) char s_x1[kATile];
    __shared__ __align__(16) char s_x2[kATile];
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lr = lane & 31, h = lane >> 5;

    // level-pair table: thread t writes entry t of all 64 lane copies
    {
        const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)p.lv.q[t & 15]);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)p.lv.q[t >> 4]);
        const uint32_t e = lo | (hi << 16);
        u32x4 *row = reinterpret_cast<u32x4 *>(s_tab + 256 * t);
#pragma unroll
        for (int c = 0; c < 16; ++c) row[c] = u32x4{e, e, e, e};
    }
    const char *const tab = s_tab;
    // X tile buffer b (b a compile-time constant)
    auto xbuf = [&](auto BC) -> char * {
        constexpr int b = decltype(BC)::value;
        if constexpr (b == 0) return s_x0;
        else if constexpr (b == 1) return s_x1;
        else return s_x2;
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using B2 = std::integral_constant<int, 2>;
    const uint32_t lane4 = 4u * (uint32_t)lane;

    int64_t mt, nt;
    tile_of(blockIdx.x, (p.M + kBM - 1) / kBM, (p.N + kBN - 1) / kBN, mt, nt);
    const int64_t m0 = uniform(mt * kBM), n0 = uniform(nt * kBN);
    const int64_t K = p.K, steps = K / kBK, kb_row = K / kBlock;
    const int64_t m_rows = min((int64_t)kBM, p.M - m0), n_rows = min((int64_t)kBN, p.N - n0);

    // ---- X staging: wave w moves tile rows 64w .. 64w+63, 8 rows per load.
    // Lane l of load q fills LDS segment 64w + 8q + l/8 (which holds row
    // seg_row of it), physical chunk l % 8, which holds logical chunk
    // (l % 8) ^ (row & 7).
    const Rsrc x_rs = rsrc(p.x + m0 * K, m_rows * K * 2);
    uint32_t a_off[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = seg_row(64 * w + 8 * q + (lane >> 3));
        const int chunk = (lane & 7) ^ (row & 7);
        a_off[q] = (uint32_t)(row * K * 2 + chunk * 16);
    }
    auto stage_x = [&](const Rsrc &rs, int64_t koff_bytes, auto BC) {
        char *dst = xbuf(BC) + (64 * w) * 128;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + q * 1024), 16, a_off[q],
                                                     (int)koff_bytes, 0, 0);
    };

    // ---- W: lane (lr, h) of column tile j holds weight row n0 + 64w + 32j + lr,
    // the 32 codes of k = 32h .. 32h+31 of each step's block.
    const Rsrc c_rs = rsrc(p.codes + n0 * (K / 2), n_rows * (K / 2));
    const Rsrc q_rs = kDQ ? rsrc(p.q8 + n0 * kb_row, n_rows * kb_row)
                          : rsrc(p.absmax + n0 * kb_row, n_rows * kb_row * 4);
    const Rsrc s_rs = rsrc(p.c2, p.n_groups * 4);
    uint32_t c_off[kTN], q_off[kTN], b_abs[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        const int nl = 64 * w + 32 * j + lr;
        c_off[j] = (uint32_t)(nl * (K / 2) + 16 * h);
        q_off[j] = (uint32_t)(nl * kb_row * (kDQ ? 1 : 4));
        b_abs[j] = (uint32_t)((n0 + nl) * kb_row);
    }
    auto load_w1 = [&](int64_t s, Raw &raw, int j) {
        raw.c[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(c_rs, c_off[j],
                                                                                  (int)(s * (kBK / 2)), 0));
        if (kDQ) {
            raw.q[j] = __builtin_amdgcn_raw_buffer_load_b8(q_rs, q_off[j], (int)s, 0);
            raw.s[j] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(s_rs, ((b_abs[j] + (uint32_t)s) >> 8) * 4u, 0, 0));
        } else {
            raw.s[j] = __builtin_bit_cast(float,
                                          __builtin_amdgcn_raw_buffer_load_b32(q_rs, q_off[j], (int)(s * 4), 0));
        }
    };
    auto scale = [&](const Raw &raw, int j) {
        return kDQ ? __builtin_amdgcn_cvt_f32_fp8((int)raw.q[j], 0) * raw.s[j] : raw.s[j];
    };

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16_t{};

    // fragment read offsets: tile row 32i + lr, logical chunk 4h + ks
    uint32_t frag_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) frag_off[ks] = tile_seg(lr) * 128 + 16 * ((4 * h + ks) ^ (lr & 7));
    auto frag = [&](const char *a_t, int pr) {  // pair pr = 8 ks + i
        return *reinterpret_cast<const u32x4 *>(a_t + frag_off[pr / kTM] + (pr % kTM) * 4096);
    };

    // W operands of substeps with even (bw[0]) and odd (bw[1]) index.
    u32x4 bw[2][kTN];
    u32x4 af[kFragRing];
    float sc_c[kTN], sc_n[kTN];  // c1' of this step's and the next step's blocks

    // One K-step: 64 MFMA slots, scheduled by hand (in-order issue, one wave
    // per SIMD). Slot m issues MFMA (row tile i, column tile j) of substep
    // ks = m / 16, i = (m % 16) / 2, j = m % 2, and around it:
    //  - even slots: the X fragment kFragAhead pairs ahead;
    //  - slots 0..7 of a substep: the level read of unit u (column tile u / 4,
    //    code byte u % 4) of the next substep's W operands; slots 8..15: that
    //    unit's arithmetic into the operand;
    //  - the loads of the step after next (X tile part q at slot 6q + 3, the
    //    codes of column tile j at slot 12j + 1) and, at kBarrierSlot, the
    //    wait for this wave's part of the next X tile plus a barrier.
    constexpr int kLoadsPerStep = 8 + (kDQ ? 3 : 2) * kTN;
    auto step = [&](int64_t s, auto BC, const Raw &rc, const Raw &rn, Raw &rl) {
        constexpr int b = decltype(BC)::value;  // s % 3
        const char *a_t = xbuf(std::integral_constant<int, b>{});
        const char *a_next = xbuf(std::integral_constant<int, (b + 1) % 3>{});
        char *const x_dst = xbuf(std::integral_constant<int, (b + 2) % 3>{}) + (64 * w) * 128;
        const int64_t sl = min(s + 2, steps - 1);
        uint32_t lq[kUnits];
#pragma clang loop unroll(full)
        for (int m = 0; m < 2 * kPairs; ++m) {
            const int ks = m / 16, sm = m % 16, i = sm / 2, j = sm % 2, pr = m / 2;
            if (m == kBarrierSlot) {
                // This wave's part of the next X tile (loaded during step s-1)
                // has landed and its reads of earlier tiles are done; the
                // barrier makes that true of every wave. A plain s_barrier: the
                // fence of __syncthreads would also wait for this step's tile.
                __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kLoadsPerStep) & ~(0xF << 8));
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            if (m % 2 == 0) {
                u32x4 &dst = af[(pr + kFragAhead) % kFragRing];
                if (pr + kFragAhead < kPairs)
                    dst = frag(a_t, pr + kFragAhead);
                else
                    dst = frag(a_next, pr + kFragAhead - kPairs);
            }
            if (m % 6 == 3 && m / 6 < 8) {
                const int q = m / 6;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rs, (lds_void *)(x_dst + q * 1024), 16, a_off[q],
                                                         (int)(sl * (kBK * 2)), 0, 0);
            }
            if (m % 12 == 1 && m / 12 < kTN) load_w1(sl, rl, m / 12);
            // W operands of substep ks + 1 (of the next step's substep 0 in
            // substep 3): level reads in slots 0..7, arithmetic in 8..15
            if (sm < kUnits) {
                const int u = sm, uj = u / 4, uh = u % 4;
                if (ks == 3 && uh == 0) sc_n[uj] = scale(rn, uj);
                const uint32_t d = (ks < 3) ? rc.c[uj][ks + 1] : rn.c[uj][0];
                lq[u] = level_pair(tab, d, uh, lane4);
            } else {
                const int u = sm - kUnits, uj = u / 4, uh = u % 4;
                const float sc = (ks < 3) ? sc_c[uj] : sc_n[uj];
                bw[(ks + 1) % 2][uj][uh] = scale_pair(lq[u], sc);
            }
            mfma32(acc[i][j], af[pr % kFragRing], bw[ks % 2][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int jj = 0; jj < kTN; ++jj) sc_c[jj] = sc_n[jj];
    };

    // ---- main loop over the NF4 segment. X tiles are staged two steps ahead
    // into 3 LDS buffers and codes two steps ahead into 3 register slots; one
    // barrier per step, at kBarrierSlot. The loop is unrolled by 3 so that
    // every buffer and slot index is a compile-time constant.
    Raw r0, r1, r2;
    stage_x(x_rs, 0, B0{});
    stage_x(x_rs, min((int64_t)1, steps - 1) * (kBK * 2), B1{});
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        load_w1(0, r0, j);
        load_w1(min((int64_t)1, steps - 1), r1, j);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // pair table, X tiles 0 and 1
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        sc_c[j] = scale(r0, j);
        sc_n[j] = sc_c[j];
#pragma unroll
        for (int uh = 0; uh < 4; ++uh) bw[0][j][uh] = scale_pair(level_pair(tab, r0.c[j][0], uh, lane4), sc_c[j]);
    }
#pragma unroll
    for (int f = 0; f < kFragAhead; ++f) af[f] = frag(xbuf(B0{}), f);
    valu_to_mfma();
    int64_t s = 0;
    for (; s + 3 <= steps; s += 3) {
        step(s, B0{}, r0, r1, r2);
        step(s + 1, B1{}, r1, r2, r0);
        step(s + 2, B2{}, r2, r0, r1);
    }
    if (s < steps) step(s++, B0{}, r0, r1, r2);
    if (s < steps) step(s++, B1{}, r1, r2, r0);
    __builtin_amdgcn_s_waitcnt(0);  // the clamped tail loads
    __syncthreads();

    // ---- adapter segment: + T' . B over rp / 64 steps (not pipelined)
    if (p.t != nullptr) {
        const Rsrc t_rs = rsrc(p.t + m0 * p.rp, m_rows * p.rp * 2);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int row = seg_row(64 * w + 8 * q + (lane >> 3));
            const int chunk = (lane & 7) ^ (row & 7);
            a_off[q] = (uint32_t)(row * p.rp * 2 + chunk * 16);
        }
        for (int64_t sa = 0; sa < p.rp / kBK; ++sa) {
            stage_x(t_rs, sa * (kBK * 2), B0{});
            // B operand of lane (lr, h), column tile j, substep ks: B[k][n],
            // k = 64 sa + 32 h + 8 ks + e (the K order of the NF4 segment)
            u32x4 ba[4][kTN];
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int64_t n = min(n0 + 64 * w + 32 * j + lr, p.N - 1);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    uint32_t d[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; ++e2) {
                        const int64_t k = 64 * sa + 32 * h + 8 * ks + 2 * e2;
                        const uint32_t lo = (k < p.r) ? p.b[k * p.N + n] : 0u;
                        const uint32_t hi = (k + 1 < p.r) ? p.b[(k + 1) * p.N + n] : 0u;
                        d[e2] = lo | (hi << 16);
                    }
                    ba[ks][j] = u32x4{d[0], d[1], d[2], d[3]};
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            valu_to_mfma();
#pragma unroll
            for (int pr = 0; pr < kPairs; ++pr) {
                const u32x4 a = frag(xbuf(B0{}), pr);
#pragma unroll
                for (int j = 0; j < kTN; ++j) mfma32(acc[pr % kTM][j], a, ba[pr / kTM][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
            mfma_drain();  // before the next iteration rewrites the operands
            __syncthreads();
        }
    }

    // ---- the accumulators are final once the last MFMA has drained; the
    // statements below tie every accumulator to a point after that wait, so
    // no read of them (AGPR to VGPR copies included) is placed earlier.
    mfma_drain();
#pragma unroll
    for (int i = 0; i < kTM; ++i) asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]));

    // ---- epilogue: the bf16 results go through LDS so that each lane stores
    // 16 contiguous bytes. Wave w stages its 256 x 64 slice (32 KiB, rows of
    // 128 B, 16-byte chunks XOR-swizzled by row / 4) in the table's two
    // halves (waves 0, 1) and X tiles 0, 1 (waves 2, 3), all dead by now.
    // Accumulator v of tile (i, j) in lane (lr, h) is row 32i + 8(v/4) + 4h +
    // v % 4, column 32j + lr.
    __syncthreads();
    {
        char *const ep = w < 2 ? s_tab + w * 32768 : (w == 2 ? s_x0 : s_x1);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 32 * i + 8 * (v / 4) + 4 * h + v % 4, col = 32 * j + lr;
                    const int chunk = (col >> 3) ^ ((row >> 2) & 7);
                    *reinterpret_cast<uint16_t *>(ep + row * 128 + chunk * 16 + (col & 7) * 2) =
                        (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xFFFFu);
                }
        __syncthreads();
        const int64_t col0 = n0 + 64 * w;
        if (col0 < p.N) {
#pragma unroll 4
            for (int it = 0; it < 32; ++it) {
                const int row = 8 * it + (lane >> 3), c = lane & 7;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(ep + row * 128 + 16 * (c ^ ((row >> 2) & 7)));
                if (m0 + row < p.M)
                    *reinterpret_cast<u32x4 *>(p.y + (m0 + row) * p.N + col0 + 8 * c) = v;
            }
        }
    }
}

template <bool kDQ>
hipError_t run_fwd(const FwdParams &p, hipStream_t s) {
    const int64_t tiles = ((p.M + kBM - 1) / kBM) * ((p.N + kBN - 1) / kBN);
    gemm_fwd_kernel<kDQ><<<dim3((unsigned)tiles), dim3(kThreads), 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

bool fwd_main_supported(int64_t k) { return k <= (1 << 22); }

// Y = X . W'^T (+ T' . B when t != nullptr). K % 64 == 0, N % 64 == 0,
// K <= 2^22 (each per-tile buffer descriptor spans under 4 GiB).
hipError_t launch_fwd_main(const uint16_t *x, int64_t m, const nf4_weight &w, const uint16_t *t,
                           int64_t rp, const uint16_t *b, int32_t r, uint16_t *y, hipStream_t s) {
    FwdParams p{};
    p.x = x;
    p.M = m;
    p.K = w.k_in;
    p.N = w.n_out;
    p.codes = w.codes;
    p.q8 = w.absmax_q;
    p.c2 = w.absmax_scale;
    p.n_groups = (w.n_out * (w.k_in / kBlock) + kDqBlock - 1) / kDqBlock;
    p.absmax = w.absmax;
    p.t = t;
    p.rp = rp;
    p.b = b;
    p.r = r;
    p.y = y;
    p.lv = levels();
    return w.absmax_q ? run_fwd<true>(p, s) : run_fwd<false>(p, s);
}

}  // namespace nf4
