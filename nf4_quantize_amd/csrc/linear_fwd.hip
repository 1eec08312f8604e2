// linear_fwd.hip - large-M fused NF4 linear forward for gfx950 on bf16 MFMA
// ([MF] "Forward Pass Computation"; source key in nf4_internal.h):
//   Y = X . W'^T + T' . B,   T' = s (X . A) (bf16, computed beforehand),
// W' = dequantize(W), W stored [N x K] NF4 (64-blocks along K).
//
// Tile: a workgroup of 4 waves owns 256 rows x 256 columns of Y; wave w owns
// all 256 rows of columns 64w .. 64w+63, as 16 x 4 tiles of
// v_mfma_f32_16x16x32_bf16 (256 fp32 accumulators per lane, held in AGPRs).
// K advances 64 (one NF4 block) per step.
//
//  - X goes global -> LDS directly (buffer_load ... lds, no registers),
//    double buffered, rows of 128 B with 16-byte chunks XOR-swizzled by row
//    so the fragment reads of 16 rows hit distinct banks.
//  - W never touches LDS: each lane loads the 8 code bytes its MFMA operands
//    need (one weight row, 16 consecutive k) and dequantizes them in
//    registers to bf16(q[code] * c1') through a 256-entry (low, high) level
//    table in LDS, the levels held as fp16 (see level_pair). The 32 k of an MFMA are taken
//    in the order that makes a lane's 16 k of one step contiguous: lane group
//    g covers k = 16g .. 16g+15, half ks (0, 1) of it in MFMA ks. X fragments
//    are read in the same order, so the contraction is unchanged.
//  - Step s's MFMAs run while step s+1's operands are dequantized and step
//    s+1's X tile and step s+2's codes are in flight.
// All loads are raw buffer loads with per-tile descriptors whose size stops
// at the last valid row: rows beyond M or N read as zero, the loop has no
// branches, and the per-step advance is a scalar offset.
#include <utility>

#include "gemm_common.h"

namespace nf4 {
namespace {

using namespace gemm;

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kTM = kBM / 16;                // 16 row tiles per wave
constexpr int kTN = 64 / 16;                 // 4 column tiles per wave
constexpr int kATile = kBM * kBK * 2;        // 32 KiB of bf16 per X tile
constexpr int kXBufs = 3;                    // X tiles in flight: steps s, s+1, s+2
constexpr int kTable = 256 * 256;            // level-pair table, one copy per lane
constexpr int kLds = kTable + kXBufs * kATile;  // 160 KiB: table and X tiles, all static
constexpr int kFragAhead = 3;                // X fragments read this many row groups ahead
constexpr int kLookAhead = 16;               // MFMA slots between a level read and its use
constexpr int kLookRing = 8;                 // level reads in flight
// The fragment ring is indexed by the row group within a step, and the next
// step's first fragments are read at the end of the current one: the ring
// length must divide the 32 row groups of a step to keep its phase.
static_assert((2 * kTM) % (kFragAhead + 1) == 0, "fragment ring must divide a step");
constexpr int kBarrierSlot = 4 * (2 * kTM - kFragAhead);  // first slot reading the next step's tile
static_assert(kLookRing * 3 > kLookAhead, "level reads in flight exceed the ring");
static_assert(45 + kLookAhead < 64, "half-1 operands must be finished within half 0");

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


// Level-pair table in LDS: the entry of code byte b holds (q[b & 15],
// q[b >> 4]) as two fp16 (the LDS read bandwidth, not the arithmetic, bounds
// this kernel: a 4-byte entry halves the bytes of an 8-byte fp32 pair). Each
// lane has its own copy, entry b of lane l at byte 256 b + 4 l, so the 32
// lanes of each half-wave (LDS serves 32-bit reads a half-wave at a time)
// hit 32 distinct banks whatever the code bytes. For byte h of the
// code dword d, v_perm builds the address (b << 8) | 4 l in one instruction.
// The fp16 levels differ from the fp32 ones by at most 2^-12 relative, far
// below the bf16 rounding of the operand.
// The table is a static LDS array: its base folds into the read's offset.
__device__ __forceinline__ uint32_t level_pair(const char *tab, uint32_t d, int h, uint32_t lane4) {
    const uint32_t addr = __builtin_amdgcn_perm(d, lane4, 0x0C0C0400u | ((uint32_t)h << 8));
    return *reinterpret_cast<const uint32_t *>(tab + addr);
}
// 8 weights (one code dword, element e in bits 4e..4e+3) -> 4 dwords of bf16 pairs.
__device__ __forceinline__ u32x4 deq8(const char *tab, uint32_t d, float sc, uint32_t lane4) {
    u32x4 o;
#pragma unroll
    for (int h = 0; h < 4; ++h) o[h] = scale_pair(level_pair(tab, d, h, lane4), sc);
    return o;
}

// Codes and scale inputs of one K-step for a lane's 4 column tiles.
struct Raw {
    uint2 c[kTN];     // 16 codes: k = 16g .. 16g+15 of the block
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
    static_assert(kTable + 3 * kATile == kLds && kXBufs == 3, "LDS layout");
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lr = lane & 15, g = lane >> 4;

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
    // Lane l of load q fills LDS row 64w + 8q + l/8, physical chunk l % 8,
    // which holds logical chunk (l % 8) ^ ((row >> 1) & 7).
    const Rsrc x_rs = rsrc(p.x + m0 * K, m_rows * K * 2);
    uint32_t a_off[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 64 * w + 8 * q + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        a_off[q] = (uint32_t)(row * K * 2 + chunk * 16);
    }
    auto stage_x = [&](const Rsrc &rs, int64_t koff_bytes, auto BC) {
        char *dst = xbuf(BC) + (64 * w) * 128;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + q * 1024), 16, a_off[q],
                                                     (int)koff_bytes, 0, 0);
    };

    // ---- W: lane (lr, g) of column tile j holds row n0 + 64w + 16j + lr.
    const Rsrc c_rs = rsrc(p.codes + n0 * (K / 2), n_rows * (K / 2));
    const Rsrc q_rs = kDQ ? rsrc(p.q8 + n0 * kb_row, n_rows * kb_row)
                          : rsrc(p.absmax + n0 * kb_row, n_rows * kb_row * 4);
    const Rsrc s_rs = rsrc(p.c2, p.n_groups * 4);
    uint32_t c_off[kTN], q_off[kTN], b_abs[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
        const int nl = 64 * w + 16 * j + lr;
        c_off[j] = (uint32_t)(nl * (K / 2) + 8 * g);
        q_off[j] = (uint32_t)(nl * kb_row * (kDQ ? 1 : 4));
        b_abs[j] = (uint32_t)((n0 + nl) * kb_row);
    }
    auto load_w = [&](int64_t s, Raw &raw) {
#pragma unroll
        for (int j = 0; j < kTN; ++j) {
            raw.c[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(c_rs, c_off[j],
                                                                                     (int)(s * (kBK / 2)), 0));
            if (kDQ) {
                raw.q[j] = __builtin_amdgcn_raw_buffer_load_b8(q_rs, q_off[j], (int)s, 0);
                raw.s[j] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(s_rs, ((b_abs[j] + (uint32_t)s) >> 8) * 4u, 0, 0));
            } else {
                raw.s[j] = __builtin_bit_cast(float,
                                              __builtin_amdgcn_raw_buffer_load_b32(q_rs, q_off[j], (int)(s * 4), 0));
            }
        }
    };
    auto scale = [&](const Raw &raw, int j) {
        return kDQ ? __builtin_amdgcn_cvt_f32_fp8((int)raw.q[j], 0) * raw.s[j] : raw.s[j];
    };

    f32x4_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment read offsets: tile row 16i + lr, logical chunk 2g + ks
    uint32_t frag_off[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) frag_off[ks] = lr * 128 + 16 * ((2 * g + ks) ^ ((lr >> 1) & 7));
    auto frag = [&](const char *a_t, int idx) {
        return *reinterpret_cast<const u32x4 *>(a_t + frag_off[idx / kTM] + (idx % kTM) * 2048);
    };

    // B operands of the MFMA halves ks = 0 (b0) and ks = 1 (b1).
    u32x4 b0[kTN], b1[kTN];

    // One K-step, scheduled by hand at the granularity of single MFMAs so
    // that every MFMA is followed by the few other instructions that fit in
    // its shadow (in-order issue; one wave per SIMD). Slot m (0..127) issues
    // MFMA (row tile m/4 mod 16, column tile m%4, half m/64) and around it:
    //  - the X fragment of row group m/4 + 2 (slots with m%4 == 0);
    //  - the 16 code bytes of this step's half-1 operands b1 (from rc) and,
    //    in half 1, of the next step's half-0 operands b0 (from rn): one byte
    //    per 3 slots, its level pair read from LDS 8 slots before it is
    //    scaled and rounded into the operand;
    //  - the loads of the step after next (spread over the step, see below).
    // X fragments in flight; the first kFragAhead of a step are read at the end
    // of the previous step (its X tile has landed by then: each step ends with
    // the wait for the next step's tile and a barrier).
    u32x4 af[kFragAhead + 1];
    // Loads issued after the last load of step s-1 by the barrier slot of step
    // s: all of step s's (X tile and codes are issued by slot 115).
    constexpr int kLoadsPerStep = 8 + (kDQ ? 3 : 2) * kTN;
    constexpr int kAfterTile = kLoadsPerStep;
    static_assert(16 * 7 + 3 < kBarrierSlot && 32 * (kTN - 1) + 1 < kBarrierSlot, "loads before the barrier");
    auto step = [&](int64_t s, auto BC, const Raw &rc, const Raw &rn, Raw &rl) {
        constexpr int b = decltype(BC)::value;  // s % 3
        const char *a_t = xbuf(std::integral_constant<int, b>{});
        const char *a_next = xbuf(std::integral_constant<int, (b + 1) % 3>{});
        char *const x_dst = xbuf(std::integral_constant<int, (b + 2) % 3>{}) + (64 * w) * 128;
        uint32_t lq[kLookRing];
        float sc1[kTN], sc0[kTN];
#pragma clang loop unroll(full)
        for (int m = 0; m < 128; ++m) {
            const int grp = m / 4, sub = m % 4, ks = grp / kTM, i = grp % kTM;
            if (m == kBarrierSlot) {
                // This wave's part of the next step's X tile (loaded during step
                // s-1, like everything before this step's loads) has landed and
                // its reads of tiles before it are done; the
                // barrier makes that true of every wave, so the next tile can be
                // read and the tile loaded at the start of step s+1 can reuse the
                // buffer of step s-1. A plain s_barrier: the fence of
                // __syncthreads would also wait for the tile loaded during step s.
                __builtin_amdgcn_s_waitcnt(vmcnt_at_most(kAfterTile) & ~(0xF << 8));
                asm volatile("" ::: "memory");
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
            }
            if (sub == 0) {
                u32x4 &dst = af[(grp + kFragAhead) % (kFragAhead + 1)];
                if (grp + kFragAhead < 2 * kTM)
                    dst = frag(a_t, grp + kFragAhead);
                else
                    dst = frag(a_next, grp + kFragAhead - 2 * kTM);
            }
            // loads spread over the step (all four waves run this schedule in
            // step with each other, so bunched loads would meet at the memory
            // pipeline and the LDS together): part q of the next-but-one X tile
            // at slot 16q + 3, the codes of column tile j at slot 32j + 1
            if (m % 16 == 3) {
                const int q = m / 16;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(x_rs, (lds_void *)(x_dst + q * 1024), 16, a_off[q],
                                                         (int)(min(s + 2, steps - 1) * (kBK * 2)), 0, 0);
            }
            if (m % 32 == 1) {
                const int j = m / 32;
                const int64_t sl = min(s + 2, steps - 1);
                rl.c[j] = __builtin_bit_cast(
                    uint2, __builtin_amdgcn_raw_buffer_load_b64(c_rs, c_off[j], (int)(sl * (kBK / 2)), 0));
                if (kDQ) {
                    rl.q[j] = __builtin_amdgcn_raw_buffer_load_b8(q_rs, q_off[j], (int)sl, 0);
                    rl.s[j] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(s_rs, ((b_abs[j] + (uint32_t)sl) >> 8) * 4u, 0, 0));
                } else {
                    rl.s[j] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(q_rs, q_off[j], (int)(sl * 4), 0));
                }
            }
            // level reads: unit u = 4j + h is byte h of operand j
            const int hm = m % 64;
            if (hm % 3 == 0 && hm / 3 < 16) {
                const int u = hm / 3, j = u / 4, h = u % 4;
                const uint32_t d = (m < 64) ? rc.c[j].y : rn.c[j].x;
                lq[u % kLookRing] = level_pair(tab, d, h, lane4);
                if (h == 0) {
                    if (m < 64) sc1[j] = scale(rc, j);
                    else sc0[j] = scale(rn, j);
                }
            }
            if (hm >= kLookAhead && (hm - kLookAhead) % 3 == 0 && (hm - kLookAhead) / 3 < 16) {
                const int u = (hm - kLookAhead) / 3, j = u / 4, h = u % 4;
                const float sc = (m < 64) ? sc1[j] : sc0[j];
                const uint32_t v = scale_pair(lq[u % kLookRing], sc);
                if (m < 64) b1[j][h] = v;
                else b0[j][h] = v;
            }
            mfma(acc[i][sub], af[grp % (kFragAhead + 1)], ks ? b1[sub] : b0[sub]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- main loop over the NF4 segment. X tiles are staged two steps ahead
    // into 3 LDS buffers and codes two steps ahead into 3 register slots; one
    // barrier per step, at kBarrierSlot (see step). The loop is unrolled by
    // 3 so that every buffer and slot index is a compile-time constant.
    Raw r0, r1, r2;
    stage_x(x_rs, 0, B0{});
    stage_x(x_rs, min((int64_t)1, steps - 1) * (kBK * 2), B1{});
    load_w(0, r0);
    load_w(min((int64_t)1, steps - 1), r1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // pair table, X tiles 0 and 1
#pragma unroll
    for (int j = 0; j < kTN; ++j) b0[j] = deq8(tab, r0.c[j].x, scale(r0, j), lane4);
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
            const int row = 64 * w + 8 * q + (lane >> 3);
            const int chunk = (lane & 7) ^ ((row >> 1) & 7);
            a_off[q] = (uint32_t)(row * p.rp * 2 + chunk * 16);
        }
        for (int64_t sa = 0; sa < p.rp / kBK; ++sa) {
            stage_x(t_rs, sa * (kBK * 2), B0{});
            // B operand of lane (lr, g), tile j, half ks: B[k][n], k = 64sa + 16g + 8ks + e
#pragma unroll
            for (int j = 0; j < kTN; ++j) {
                const int64_t n = min(n0 + 64 * w + 16 * j + lr, p.N - 1);
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint32_t d[4];
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int64_t k = 64 * sa + 16 * g + 8 * ks + 2 * h;
                        const uint32_t lo = (k < p.r) ? p.b[k * p.N + n] : 0u;
                        const uint32_t hi = (k + 1 < p.r) ? p.b[(k + 1) * p.N + n] : 0u;
                        d[h] = lo | (hi << 16);
                    }
                    (ks ? b1[j] : b0[j]) = u32x4{d[0], d[1], d[2], d[3]};
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            valu_to_mfma();
#pragma unroll
            for (int idx = 0; idx < 2 * kTM; ++idx) {
                const int ks = idx / kTM, i = idx % kTM;
                const u32x4 a = frag(xbuf(B0{}), idx);
#pragma unroll
                for (int j = 0; j < kTN; ++j) mfma(acc[i][j], a, ks ? b1[j] : b0[j]);
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
    for (int i = 0; i < kTM; i += 2)
        asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                     "+a"(acc[i + 1][0]), "+a"(acc[i + 1][1]), "+a"(acc[i + 1][2]), "+a"(acc[i + 1][3]));

    // ---- epilogue: the bf16 results go through LDS so that each lane stores
    // 16 contiguous bytes. Wave w stages its 256 x 64 slice (32 KiB, rows of
    // 128 B, 16-byte chunks XOR-swizzled by row / 4) in the table's two
    // halves (waves 0, 1) and X tiles 0, 1 (waves 2, 3), all dead by now. D
    // element q of tile (i, j) is row 16i + 4g + q, column 16j + lr.
    __syncthreads();
    {
        char *const ep = w < 2 ? s_tab + w * 32768 : (w == 2 ? s_x0 : s_x1);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 16 * i + 4 * g + q, col = 16 * j + lr;
                    const int chunk = (col >> 3) ^ ((row >> 2) & 7);
                    *reinterpret_cast<uint16_t *>(ep + row * 128 + chunk * 16 + (col & 7) * 2) =
                        (uint16_t)(pack_bf16x2(acc[i][j][q], 0.0f) & 0xFFFFu);
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
