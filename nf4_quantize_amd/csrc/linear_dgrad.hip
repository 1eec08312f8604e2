// linear_dgrad.hip - input gradient of the fused NF4 linear for gfx950 on
// bf16 MFMA ([MF] "Gradient Computation", the activation-gradient equation;
// source key in nf4_internal.h):
//   dX = dY . W' + U' . A^T,   U' = s (dY . B^T) (bf16, computed beforehand),
// W' = dequantize(W), W stored [N x K] NF4 (64-blocks along K); the
// contraction runs over N, the rows of W.
//
// Tile: a workgroup of 4 waves owns 256 rows x 256 columns of dX; wave
// w = 2 wr + wc owns rows 128 wr .. +127 and columns 128 wc .. +127 as 8 x 8
// tiles of v_mfma_f32_16x16x32_bf16 (accumulators in AGPRs). A step contracts
// 64 rows of W (one NF4 block width of dX columns per row). W' is dequantized
// once per workgroup into an LDS tile, so the 2 x 2 split of the waves costs
// no extra dequantization; it halves the dY operand reads (each wave reads
// 128 rows, not 256) for twice the W' operand reads: per step the CU's LDS
// moves 224 KiB instead of 256 KiB.
//
//  - dY goes global -> LDS directly (buffer_load ... lds), double buffered,
//    like X in the forward kernel.
//  - The MFMA operand needs 8 consecutive contraction indices of one dX
//    column, i.e. 8 rows of W: each thread loads an 8 x 8 patch of codes
//    (8 rows of 8 columns), dequantizes it as bf16(q[code] * c1'),
//    transposes it in registers and writes 8 columns into a double-buffered
//    LDS tile [column][row]; waves read their operands from there.
//  - One barrier per step, at MFMA slot kBarrierSlot: by then this step's
//    operand reads of both buffers it will overwrite are done, the next dY
//    tile has landed and the next W tile is written; the slots after it
//    already read the next step's first operands.
#include "gemm_common.h"

namespace nf4 {
namespace {

using namespace gemm;

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kTM = 128 / 16;             // 8 row tiles per wave
constexpr int kTN = 128 / 16;             // 8 column tiles per wave
constexpr int kATile = kBM * kBK * 2;      // 32 KiB of bf16 dY per step
constexpr int kBTile = kBN * kBK * 2;      // 32 KiB of bf16 W' per step
constexpr int kTable = 256 * 32 * 4;       // level-pair table, one copy per half-wave lane
constexpr int kLds = kTable + 2 * kATile + 2 * kBTile;  // 160 KiB
constexpr int kFragAhead = 3;              // dY fragments read this many row groups ahead
constexpr int kLookAhead = 16;             // MFMA slots between a level read and its use
constexpr int kLookRing = 8;
// the first slot that reads the next step's dY tile (a row group is kTN slots)
constexpr int kBarrierSlot = kTN * (2 * kTM - kFragAhead);
static_assert(2 * kLookRing >= kLookAhead, "level reads in flight exceed the ring");
static_assert(62 + kLookAhead < 96, "the patch must be finished before it is written");
static_assert((2 * kTM) % (kFragAhead + 1) == 0, "fragment ring must divide a step");
static_assert(kTM * kTN * 2 == 128, "128 MFMA slots per step");
static_assert(32 + 10 * 7 < kBarrierSlot && 96 < kBarrierSlot, "all loads and the W' write of a step before its barrier");
static_assert(kBarrierSlot + kTN < 128, "next step's first W' operands read within the step");

struct DgradParams {
    const uint16_t *dy;     // dY [M x N]
    int64_t M, K, N;
    const uint8_t *codes;   // W codes [N x K/2]
    const uint8_t *q8;      // E4M3 codes of c1/c2 (double quantization) or nullptr
    const float *c2;
    int64_t n_groups;
    const float *absmax;    // c1 (no double quantization)
    const uint16_t *u;      // U' [M x rp] bf16, or nullptr (no adapter)
    int64_t rp;
    const uint16_t *a;      // A [K x r] bf16
    int32_t r;
    uint16_t *dx;           // dX [M x K] bf16
    Levels lv;
};

// A thread's 8 x 8 patch of W for one step: rows 8 jp + i, columns 8 cp .. 8 cp + 7.
struct Patch {
    uint32_t c[8];  // code dword of row i (8 columns)
    uint32_t q[8];  // E4M3 code of c1/c2 of row i's block
    float s[8];     // c2 (double quantization) or c1
};

// 8x8 bf16 transpose within a thread: in[i] holds row i (8 values as 4
// dwords, element e in half e & 1 of dword e >> 1), out[e] holds column e.
__device__ __forceinline__ void transpose8x8(const uint32_t (&in)[8][4], u32x4 (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = in[2 * p][e >> 1], hi = in[2 * p + 1][e >> 1];
            d[p] = (e & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u) : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
        }
        out[e] = u32x4{d[0], d[1], d[2], d[3]};
    }
}

template <bool kDQ>
__global__ __launch_bounds__(kThreads) void gemm_dgrad_kernel(DgradParams p) {
    extern __shared__ __align__(16) char smem[];
    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lr = lane & 15, g = lane >> 4;

    // level-pair table at LDS address 0 (no static LDS in this kernel): the
    // fp16 pair of code byte b for copy p at byte 128 b + 4 p. Lane l reads
    // copy l % 32: LDS serves a wave's 32-bit reads one half-wave at a time,
    // and the 32 lanes of a half-wave then read 32 distinct banks.
    {
        const uint32_t e = f16_pair(p.lv.q[t & 15], p.lv.q[t >> 4]);
        u32x4 *row = reinterpret_cast<u32x4 *>(smem + 128 * t);
#pragma unroll
        for (int c = 0; c < 8; ++c) row[c] = u32x4{e, e, e, e};
    }
    const uint32_t pair4 = 4u * (uint32_t)(lane & 31);
    auto level = [&](uint32_t d, int h) {
        const uint32_t addr = (((d >> (8 * h)) & 0xFFu) << 7) | pair4;
        return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t *>(addr);
    };
    char *const ybuf = smem + kTable;
    char *const wbuf = smem + kTable + 2 * kATile;

    int64_t mt, nt;
    tile_of(blockIdx.x, (p.M + kBM - 1) / kBM, (p.K + kBN - 1) / kBN, mt, nt);
    const int64_t m0 = uniform(mt * kBM), c0 = uniform(nt * kBN);
    const int64_t K = p.K, N = p.N, steps = N / kBK, kb_row = K / kBlock;
    const int64_t m_rows = min((int64_t)kBM, p.M - m0);

    // ---- dY staging (as X in the forward kernel), rows of N elements
    const Rsrc y_rs = rsrc(p.dy + m0 * N, m_rows * N * 2);
    uint32_t a_off[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 64 * w + 8 * q + (lane >> 3);
        const int chunk = (lane & 7) ^ ((row >> 1) & 7);
        a_off[q] = (uint32_t)(row * N * 2 + chunk * 16);
    }

    // ---- W patches: thread (jp, cp) = (t % 8, t / 8); columns beyond K read
    // as zero (the descriptors stop at the end of the arrays).
    // (descriptors are per tile, so uniform; the patch column is in the
    // per-lane offset, pushed out of range for columns beyond K)
    const int jp = t & 7, cp = t >> 3;
    const int64_t col = c0 + 8 * cp;  // first column of the patch
    const Rsrc c_rs = rsrc(p.codes + c0 / 2, (N * K - c0) / 2);
    const Rsrc q_rs = kDQ ? rsrc(p.q8 + c0 / kBlock, N * kb_row - c0 / kBlock)
                          : rsrc(p.absmax + c0 / kBlock, (N * kb_row - c0 / kBlock) * 4);
    const Rsrc s_rs = rsrc(p.c2, p.n_groups * 4);
    const bool col_ok = col < K;
    uint32_t c_off[8], q_off[8], b_abs[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t jr = 8 * jp + i;  // row within the step
        c_off[i] = col_ok ? (uint32_t)(jr * (K / 2) + 4 * cp) : 0xFFFFFFF0u;
        q_off[i] = col_ok ? (uint32_t)((jr * kb_row + (cp >> 3)) * (kDQ ? 1 : 4)) : 0xFFFFFFF0u;
        b_abs[i] = (uint32_t)(jr * kb_row + col / kBlock);
    }
    auto load_patch = [&](int64_t s, Patch &pt) {
        const int64_t j0 = s * kBK;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            pt.c[i] = __builtin_amdgcn_raw_buffer_load_b32(c_rs, c_off[i], (int)(j0 * (K / 2)), 0);
            if (kDQ) {
                pt.q[i] = __builtin_amdgcn_raw_buffer_load_b8(q_rs, q_off[i], (int)(j0 * kb_row), 0);
                pt.s[i] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(
                               s_rs, ((b_abs[i] + (uint32_t)(j0 * kb_row)) >> 8) * 4u, 0, 0));
            } else {
                pt.s[i] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(q_rs, q_off[i], (int)(j0 * kb_row * 4), 0));
            }
        }
    };
    auto scale = [&](const Patch &pt, int i) {
        return kDQ ? __builtin_amdgcn_cvt_f32_fp8((int)pt.q[i], 0) * pt.s[i] : pt.s[i];
    };
    // W tile layout: row c (0..255) of 64 contraction values, 128 B, 16-byte
    // chunks XOR-swizzled by (c >> 1) & 7; the patch's column e goes to row
    // 8 cp + e, chunk jp.
    auto write_patch = [&](const uint32_t (&rows)[8][4], int buf) {
        u32x4 cols[8];
        transpose8x8(rows, cols);
        char *dst = wbuf + buf * kBTile;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cp + e;
            *reinterpret_cast<u32x4 *>(dst + c * 128 + 16 * (jp ^ ((c >> 1) & 7))) = cols[e];
        }
    };

    // ---- MFMA operands: dY tile row 128 wr + 16 i + lr and W tile row
    // 128 wc + 16 jt + lr, logical chunk 2g + ks (the swizzle of such a row is
    // (lr >> 1) & 7)
    const int wr = w >> 1, wc = w & 1;
    uint32_t frag_off[2], bfrag_off[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        frag_off[ks] = (128 * wr + lr) * 128 + 16 * ((2 * g + ks) ^ ((lr >> 1) & 7));
        bfrag_off[ks] = (128 * wc + lr) * 128 + 16 * ((2 * g + ks) ^ ((lr >> 1) & 7));
    }
    auto afrag = [&](const char *a_t, int idx) {
        return *reinterpret_cast<const u32x4 *>(a_t + frag_off[idx / kTM] + (idx % kTM) * 2048);
    };
    auto bfrag = [&](const char *b_t, int jt, int ks) {
        return *reinterpret_cast<const u32x4 *>(b_t + bfrag_off[ks] + jt * 2048);
    };

    f32x4_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4 af[kFragAhead + 1];
    u32x4 bq0[kTN], bq1[kTN];  // B operands of halves 0 and 1

    // One step s: 128 MFMA slots (row group grp = m / 8 of dY operands, W'
    // column tile m % 8) with, around them,
    // the dY tile s+1 DMA, the patch loads of step s+2, the dequantization,
    // transpose and LDS write of step s+1's patch (from pc), the barrier, and
    // the first operands of step s+1.
    auto step = [&](int64_t s, const Patch &pc, Patch &pl) {
        const int cur = (int)(s & 1), nxt = cur ^ 1;
        const char *a_t = ybuf + cur * kATile;
        const char *a_n = ybuf + nxt * kATile;
        const char *b_t = wbuf + cur * kBTile;
        const char *b_n = wbuf + nxt * kBTile;
        uint32_t rows[8][4];
        uint32_t lq[kLookRing];
        float sc[8];
#pragma clang loop unroll(full)
        for (int m = 0; m < 128; ++m) {
            const int grp = m / kTN, sub = m % kTN, ks = grp / kTM, i = grp % kTM;
            if (m == kBarrierSlot) {
                // dY tile s+1 has landed (only this step's patch loads may be
                // in flight), W tile s+1 is written, and every read of the
                // buffers step s+1 overwrites is done
                __builtin_amdgcn_s_waitcnt(vmcnt_at_most(8 * (kDQ ? 3 : 2)));
                __syncthreads();
            }
            // loads spread over the step (the four waves run this schedule in
            // step, so bunched loads would meet at the memory pipeline
            // together): part q of dY tile s+1 at slot 4q + 1, then the patch
            // row r8 of step s+2 at slot 32 + 10 r8, all before the barrier.
            // The W' operands of half 1 are read at slots 16 .. 23 (used from
            // slot 64), those of the next step's half 0 right after the barrier.
            if (m % 4 == 1 && m / 4 < 8) {
                const int q = m / 4;
                char *dst = ybuf + nxt * kATile + (64 * w) * 128;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(y_rs, (lds_void *)(dst + q * 1024), 16, a_off[q],
                                                         (int)(min(s + 1, steps - 1) * (kBK * 2)), 0, 0);
            }
            if (m >= 32 && (m - 32) % 10 == 0 && (m - 32) / 10 < 8) {
                // patch loads of step s+2, one row per slot
                const int r8 = (m - 32) / 10;
                const int64_t j0 = min(s + 2, steps - 1) * kBK;
                pl.c[r8] = __builtin_amdgcn_raw_buffer_load_b32(c_rs, c_off[r8], (int)(j0 * (K / 2)), 0);
                if (kDQ) {
                    pl.q[r8] = __builtin_amdgcn_raw_buffer_load_b8(q_rs, q_off[r8], (int)(j0 * kb_row), 0);
                    pl.s[r8] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(
                                   s_rs, ((b_abs[r8] + (uint32_t)(j0 * kb_row)) >> 8) * 4u, 0, 0));
                } else {
                    pl.s[r8] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(q_rs, q_off[r8], (int)(j0 * kb_row * 4), 0));
                }
            }
            if (m >= 16 && m < 16 + kTN) bq1[m - 16] = bfrag(b_t, m - 16, 1);
            if (m > kBarrierSlot && m <= kBarrierSlot + kTN) bq0[m - kBarrierSlot - 1] = bfrag(b_n, m - kBarrierSlot - 1, 0);
            // dY fragments: this step's before the barrier, the next step's
            // first ones after it
            if (sub == 0) {
                u32x4 &dst = af[(grp + kFragAhead) % (kFragAhead + 1)];
                if (grp + kFragAhead < 2 * kTM)
                    dst = afrag(a_t, grp + kFragAhead);
                else
                    dst = afrag(a_n, grp + kFragAhead - 2 * kTM);
            }
            // patch of step s+1: unit u = 4 r + h is code byte h of row r; its
            // level read at slot 2u, its arithmetic kLookAhead slots later
            // (before the read that reuses its ring entry)
            if (m >= kLookAhead && (m - kLookAhead) % 2 == 0 && (m - kLookAhead) / 2 < 32) {
                const int u = (m - kLookAhead) / 2, r8 = u / 4, h = u % 4;
                rows[r8][h] = scale_pair(lq[u % kLookRing], sc[r8]);
            }
            if (m % 2 == 0 && m / 2 < 32) {
                const int u = m / 2, r8 = u / 4, h = u % 4;
                if (h == 0) sc[r8] = scale(pc, r8);
                lq[u % kLookRing] = level(pc.c[r8], h);
            }
            if (m == 96) write_patch(rows, nxt);
            mfma(acc[i][sub], af[grp % (kFragAhead + 1)], ks ? bq1[sub] : bq0[sub]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- prologue: dY tile 0, patches 0 and 1, W tile 0, first operands
    Patch pa, pb;
    {
        char *dst = ybuf + (64 * w) * 128;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(y_rs, (lds_void *)(dst + q * 1024), 16, a_off[q], 0, 0, 0);
    }
    load_patch(0, pa);
    load_patch(min((int64_t)1, steps - 1), pb);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // table
    {
        uint32_t rows[8][4];
#pragma unroll
        for (int r8 = 0; r8 < 8; ++r8) {
            const float s8 = scale(pa, r8);
#pragma unroll
            for (int h = 0; h < 4; ++h) rows[r8][h] = scale_pair(level(pa.c[r8], h), s8);
        }
        write_patch(rows, 0);
    }
    __syncthreads();  // W tile 0
#pragma unroll
    for (int f = 0; f < kFragAhead; ++f) af[f] = afrag(ybuf, f);
#pragma unroll
    for (int j = 0; j < kTN; ++j) bq0[j] = bfrag(wbuf, j, 0);
    valu_to_mfma();

    // ---- main loop: step s consumes the patch of s+1 and loads that of s+2
    int64_t s = 0;
    for (; s + 2 <= steps; s += 2) {
        step(s, pb, pa);
        step(s + 1, pa, pb);
    }
    if (s < steps) step(s, pb, pa);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- adapter segment: + U' . A^T over rp / 64 steps (not pipelined).
    // B operand of lane (lr, g), tile jt, half ks: A[c][k] for 8 consecutive
    // k = 64 sa + 16 g + 8 ks + e (rows of A are contiguous in k).
    if (p.u != nullptr) {
        const Rsrc u_rs = rsrc(p.u + m0 * p.rp, m_rows * p.rp * 2);
        uint32_t u_off[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int row = 64 * w + 8 * q + (lane >> 3);
            const int chunk = (lane & 7) ^ ((row >> 1) & 7);
            u_off[q] = (uint32_t)(row * p.rp * 2 + chunk * 16);
        }
        for (int64_t sa = 0; sa < p.rp / kBK; ++sa) {
            char *dst = ybuf + (64 * w) * 128;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(u_rs, (lds_void *)(dst + q * 1024), 16, u_off[q],
                                                         (int)(sa * (kBK * 2)), 0, 0);
#pragma unroll
            for (int jt = 0; jt < kTN; ++jt) {
                const int64_t c = c0 + 128 * wc + 16 * jt + lr;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int64_t k = 64 * sa + 16 * g + 8 * ks;
                    u32x4 v = u32x4{0, 0, 0, 0};
                    if (c < K && k < p.r) v = *reinterpret_cast<const u32x4 *>(p.a + c * p.r + k);
                    (ks ? bq1[jt] : bq0[jt]) = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            valu_to_mfma();
#pragma unroll
            for (int idx = 0; idx < 2 * kTM; ++idx) {
                const int ks = idx / kTM, i = idx % kTM;
                const u32x4 a = afrag(ybuf, idx);
#pragma unroll
                for (int jt = 0; jt < kTN; ++jt) mfma(acc[i][jt], a, ks ? bq1[jt] : bq0[jt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            mfma_drain();
            __syncthreads();
        }
    }

    // ---- accumulators final (see the forward kernel), then the epilogue
    mfma_drain();
#pragma unroll
    for (int i = 0; i < kTM; ++i)
        asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]),
                     "+a"(acc[i][4]), "+a"(acc[i][5]), "+a"(acc[i][6]), "+a"(acc[i][7]));
    __syncthreads();
    {
        // the wave's 128 x 128 bf16 block through LDS: row stride 256 B,
        // 16-byte chunks XOR-swizzled by row, then 16-byte stores along rows
        char *const ep = smem + w * 32768;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int row = 16 * i + 4 * g + q, cc = 16 * j + lr;
                    const int chunk = (cc >> 3) ^ ((row >> 2) & 15);
                    *reinterpret_cast<uint16_t *>(ep + row * 256 + chunk * 16 + (cc & 7) * 2) =
                        (uint16_t)(pack_bf16x2(acc[i][j][q], 0.0f) & 0xFFFFu);
                }
        __syncthreads();
        const int64_t rw = m0 + 128 * wr, colw = c0 + 128 * wc;
        const int c = lane & 15;
        if (colw + 8 * c < K) {
#pragma unroll 4
            for (int it = 0; it < 32; ++it) {
                const int row = 4 * it + (lane >> 4);
                const u32x4 v = *reinterpret_cast<const u32x4 *>(ep + row * 256 + 16 * (c ^ ((row >> 2) & 15)));
                if (rw + row < p.M) *reinterpret_cast<u32x4 *>(p.dx + (rw + row) * K + colw + 8 * c) = v;
            }
        }
    }
}

template <bool kDQ>
hipError_t run_dgrad(const DgradParams &p, hipStream_t s) {
    const int64_t tiles = ((p.M + kBM - 1) / kBM) * ((p.K + kBN - 1) / kBN);
    auto kern = gemm_dgrad_kernel<kDQ>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    kern<<<dim3((unsigned)tiles), dim3(kThreads), kLds, s>>>(p);
    return hipGetLastError();
}

}  // namespace

// The per-step code offsets are scalar 32-bit offsets into the codes array.
bool dgrad_main_supported(int64_t n, int64_t k) { return n * k / 2 < ((int64_t)1 << 31) && k % 64 == 0; }

// dX = dY . W' (+ U' . A^T when u != nullptr). N % 64 == 0, K % 64 == 0.
hipError_t launch_dgrad_main(const uint16_t *dy, int64_t m, const nf4_weight &w, const uint16_t *u,
                             int64_t rp, const uint16_t *a, int32_t r, uint16_t *dx, hipStream_t s) {
    DgradParams p{};
    p.dy = dy;
    p.M = m;
    p.K = w.k_in;
    p.N = w.n_out;
    p.codes = w.codes;
    p.q8 = w.absmax_q;
    p.c2 = w.absmax_scale;
    p.n_groups = (w.n_out * (w.k_in / kBlock) + kDqBlock - 1) / kDqBlock;
    p.absmax = w.absmax;
    p.u = u;
    p.rp = rp;
    p.a = a;
    p.r = r;
    p.dx = dx;
    p.lv = levels();
    return w.absmax_q ? run_dgrad<true>(p, s) : run_dgrad<false>(p, s);
}

}  // namespace nf4
