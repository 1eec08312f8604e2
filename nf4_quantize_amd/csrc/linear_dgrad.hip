// linear_dgrad.hip - input gradient of the fused NF4 linear for gfx950 on
// bf16 MFMA ([MF] "Gradient Computation", the activation-gradient equation;
// source key in nf4_internal.h):
//   dX = dY . W' + U' . A^T,   U' = s (dY . B^T) (bf16, computed beforehand),
// W' = dequantize(W), W stored [N x K] NF4 (64-blocks along K); the
// contraction runs over N, the rows of W.
//
// Tile: a workgroup of 4 waves owns 256 rows x 256 columns of dX; wave
// w = 2 wr + wc owns rows 128 wr .. +127 and columns 128 wc .. +127 as 4 x 4
// tiles of v_mfma_f32_32x32x16_bf16 (accumulators in AGPRs). A step contracts
// 64 rows of W (one NF4 block width of dX columns per row), in 4 substeps of
// 16. The 32 x 32 form issues half the MFMAs of the 16 x 16 one for the same
// work, each hiding about three times the other instructions (see the
// forward kernel), and the dequantization, transposition and LDS traffic of
// the W' tile then fit in its shadow. W' is dequantized
// once per workgroup into an LDS tile, so the 2 x 2 split of the waves costs
// no extra dequantization; it halves the dY operand reads (each wave reads
// 128 rows, not 256) for twice the W' operand reads: per step the CU's LDS
// moves 224 KiB instead of 256 KiB.
//
//  - dY goes global -> LDS directly (buffer_load ... lds), double buffered,
//    like X in the forward kernel (the tile_seg layout of gemm_common.h).
//  - The MFMA operand needs 8 consecutive contraction indices of one dX
//    column, i.e. 8 rows of W: each thread loads an 8 x 8 patch of codes
//    (8 rows of 8 columns), dequantizes it as bf16(q[code] * c1'),
//    transposes it in registers and writes 8 columns into a double-buffered
//    LDS tile [column][row]; waves read their operands from there.
//  - K order: within a step, lane half h covers contraction indices
//    32 h .. 32 h + 31 (substep ks: 32 h + 8 ks .. + 7) of both operands, so
//    an operand fragment is one 16-byte chunk of a tile row.
//  - One barrier per step, at MFMA slot kBarrierSlot: by then this step's
//    operand reads of both buffers it will overwrite are done, the next dY
//    tile has landed and the next W tile is written; the slots after it
//    already read the next step's first operands.
#include "gemm_common.h"

namespace nf4 {
namespace {

using namespace gemm;

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kTM = 128 / 32;             // 4 row tiles per wave
constexpr int kTN = 128 / 32;             // 4 column tiles per wave
constexpr int kSlots = 4 * kTM * kTN;      // 64 MFMA slots per step (4 substeps)
constexpr int kATile = kBM * kBK * 2;      // 32 KiB of bf16 dY per step
constexpr int kBTile = kBN * kBK * 2;      // 32 KiB of bf16 W' per step
constexpr int kTable = 256 * 32 * 4;       // level-pair table, one copy per half-wave lane
constexpr int kLds = kTable + 2 * kATile + 2 * kBTile;  // 160 KiB
constexpr int kFragAhead = 8;              // operand reads this many slots before their first use
constexpr int kLookAhead = 8;              // slots between a level read and its arithmetic
constexpr int kLookRing = 8;
constexpr int kPatchWrite = 40;            // first slot of the W' patch transposition and write
// the first slot that reads the next step's tiles
constexpr int kBarrierSlot = kSlots - kFragAhead;
static_assert(kLookRing >= kLookAhead, "level reads in flight exceed the ring");
static_assert(31 + kLookAhead < kPatchWrite, "the patch must be finished before it is written");
static_assert(kPatchWrite + 8 <= kBarrierSlot, "the W' write of a step before its barrier");
static_assert(2 * 7 + 1 < kBarrierSlot && 17 + 3 * 7 < kBarrierSlot, "all loads of a step before its barrier");
static_assert(kFragAhead == 8, "operand reads: slots 16 ks + {0..4, 8, 12} - 8");

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

// A thread's 8 x 8 patch of W for one step: rows 8 jp + i, columns 8 cp .. 8 cp + 7,
// and the scale data of one row of the step (lane l: row l, in the wave's block).
struct Patch {
    uint32_t c[8];  // code dword of row i (8 columns)
    uint32_t q;     // E4M3 code of c1/c2 of row `lane`
    float s;        // c2 (double quantization) or c1 of row `lane`
};

__device__ __forceinline__ void mfma32(f32x16_t &c, const u32x4 &a, const u32x4 &b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}

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
    const int lr = lane & 31, h = lane >> 5;

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
        const int row = seg_row(64 * w + 8 * q + (lane >> 3));
        const int chunk = (lane & 7) ^ (row & 7);
        a_off[q] = (uint32_t)(row * N * 2 + chunk * 16);
    }

    // ---- W patches: thread (jp, cp) = (t % 8, t / 8); columns beyond K read
    // as zero (the descriptors stop at the end of the arrays). The 64 columns
    // of wave w's patches are block w of the tile, so the wave needs one
    // scale per row of the step: lane l loads that of row l and the patch
    // rows take theirs with ds_bpermute (two loads per step, not sixteen).
    // (descriptors are per tile, so uniform; the patch column is in the
    // per-lane offset, pushed out of range for columns beyond K)
    const int jp = t & 7, cp = t >> 3;
    const int64_t col = c0 + 8 * cp;  // first column of the patch
    const Rsrc c_rs = rsrc(p.codes + c0 / 2, (N * K - c0) / 2);
    const Rsrc q_rs = kDQ ? rsrc(p.q8 + c0 / kBlock, N * kb_row - c0 / kBlock)
                          : rsrc(p.absmax + c0 / kBlock, (N * kb_row - c0 / kBlock) * 4);
    const Rsrc s_rs = rsrc(p.c2, p.n_groups * 4);
    const bool col_ok = col < K;
    uint32_t c_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t jr = 8 * jp + i;  // row within the step
        c_off[i] = col_ok ? (uint32_t)(jr * (K / 2) + 4 * cp) : 0xFFFFFFF0u;
    }
    // the scale of row `lane` of the step, block w of the tile (out of range,
    // so zero, for a block beyond K: its patches' weights are then zero)
    const bool blk_ok = c0 + kBlock * w < K;
    const uint32_t q_off = blk_ok ? (uint32_t)((lane * kb_row + w) * (kDQ ? 1 : 4)) : 0xFFFFFFF0u;
    const uint32_t b_abs = (uint32_t)(lane * kb_row + c0 / kBlock + w);
    auto load_scale = [&](int64_t j0, Patch &pt) {
        if (kDQ) {
            pt.q = __builtin_amdgcn_raw_buffer_load_b8(q_rs, q_off, (int)(j0 * kb_row), 0);
            pt.s = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(s_rs, ((b_abs + (uint32_t)(j0 * kb_row)) >> 8) * 4u, 0, 0));
        } else {
            pt.s = __builtin_bit_cast(float,
                                      __builtin_amdgcn_raw_buffer_load_b32(q_rs, q_off, (int)(j0 * kb_row * 4), 0));
        }
    };
    auto load_patch = [&](int64_t s, Patch &pt) {
        const int64_t j0 = s * kBK;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            pt.c[i] = __builtin_amdgcn_raw_buffer_load_b32(c_rs, c_off[i], (int)(j0 * (K / 2)), 0);
        load_scale(j0, pt);
    };
    // c1' of row `lane`; the scale of patch row i comes from lane 8 jp + i
    auto own_scale = [&](const Patch &pt) {
        return kDQ ? __builtin_amdgcn_cvt_f32_fp8((int)pt.q, 0) * pt.s : pt.s;
    };
    auto row_scale = [&](float own, int i) {
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (8 * jp + i), __builtin_bit_cast(int, own)));
    };
    // W tile layout: row c (0..255) of 64 contraction values, 128 B, in the
    // tile_seg layout (gemm_common.h); the patch's column e goes to row
    // 8 cp + e, chunk jp. The 8 lanes of an octet write one row's segment,
    // and octets 2k, 2k+1 (rows c, c + 8) opposite halves of the banks.
    auto write_patch = [&](const uint32_t (&rows)[8][4], int buf) {
        u32x4 cols[8];
        transpose8x8(rows, cols);
        char *dst = wbuf + buf * kBTile;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cp + e;
            *reinterpret_cast<u32x4 *>(dst + tile_seg(c) * 128 + 16 * (jp ^ (c & 7))) = cols[e];
        }
    };

    // ---- MFMA operands: lane (lr, h) reads dY tile row 128 wr + 32 i + lr and
    // W' tile row 128 wc + 32 jt + lr, logical chunk 4 h + ks (tile_seg layout:
    // such a row is in segment (its 32-row base) + tile_seg(lr), chunks
    // swizzled by lr & 7)
    const int wr = w >> 1, wc = w & 1;
    uint32_t afrag_off[4], bfrag_off[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const uint32_t in_row = 16u * (uint32_t)((4 * h + ks) ^ (lr & 7));
        afrag_off[ks] = (uint32_t)(128 * wr + tile_seg(lr)) * 128u + in_row;
        bfrag_off[ks] = (uint32_t)(128 * wc + tile_seg(lr)) * 128u + in_row;
    }
    auto afrag = [&](const char *a_t, int ks, int i) {
        return *reinterpret_cast<const u32x4 *>(a_t + afrag_off[ks] + i * 4096);
    };
    auto bfrag = [&](const char *b_t, int ks, int jt) {
        return *reinterpret_cast<const u32x4 *>(b_t + bfrag_off[ks] + jt * 4096);
    };

    f32x16_t acc[kTM][kTN];
#pragma unroll
    for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = f32x16_t{};

    // operands of substeps with even (index 0) and odd (index 1) ks
    u32x4 fa[2][kTM], fb[2][kTN];

    // One step s: 64 MFMA slots; slot m issues MFMA (row tile i, column tile
    // jt) of substep ks = m / 16, i = (m % 16) / 4, jt = m % 4, and around it:
    //  - the operand reads kFragAhead slots before their first use (slot
    //    16 ks + jt for B, 16 ks + 4 i for A; the next step's first ones, from
    //    the other buffers, after the barrier);
    //  - the dY tile s+1 DMA (part q at slot 2q + 1) and the patch loads of
    //    step s+2 (row r at slot 17 + 3r, the scale with row 0);
    //  - the dequantization of step s+1's patch (unit u = 4 r + byte: level
    //    read at slot u, arithmetic kLookAhead slots later), its transposition
    //    and LDS write from slot kPatchWrite;
    //  - the barrier at kBarrierSlot.
    auto step = [&](int64_t s, const Patch &pc, Patch &pl) {
        const int cur = (int)(s & 1), nxt = cur ^ 1;
        const char *a_t = ybuf + cur * kATile;
        const char *a_n = ybuf + nxt * kATile;
        const char *b_t = wbuf + cur * kBTile;
        const char *b_n = wbuf + nxt * kBTile;
        uint32_t rows[8][4];
        uint32_t lq[kLookRing];
        float sc[8], own = 0.0f;
        u32x4 cols[8];
#pragma clang loop unroll(full)
        for (int m = 0; m < kSlots; ++m) {
            const int ks = m / 16, sm = m % 16, i = sm / 4, jt = sm % 4;
            if (m == kBarrierSlot) {
                // dY tile s+1 has landed (only this step's patch loads may be
                // in flight), W tile s+1 is written, and every read of the
                // buffers step s+1 overwrites is done
                __builtin_amdgcn_s_waitcnt(vmcnt_at_most(8 + (kDQ ? 2 : 1)));
                __syncthreads();
            }
            // operand reads for slot m + kFragAhead
            {
                const int tm = m + kFragAhead, tks = (tm / 16) % 4, tsm = tm % 16;
                const char *at = tm < kSlots ? a_t : a_n;
                const char *bt = tm < kSlots ? b_t : b_n;
                if (tsm < 4) fb[tks & 1][tsm] = bfrag(bt, tks, tsm);
                if (tsm % 4 == 0) fa[tks & 1][tsm / 4] = afrag(at, tks, tsm / 4);
            }
            if (m % 2 == 1 && m / 2 < 8) {
                const int q = m / 2;
                char *dst = ybuf + nxt * kATile + (64 * w) * 128;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(y_rs, (lds_void *)(dst + q * 1024), 16, a_off[q],
                                                         (int)(min(s + 1, steps - 1) * (kBK * 2)), 0, 0);
            }
            if (m >= 17 && (m - 17) % 3 == 0 && (m - 17) / 3 < 8) {
                // patch loads of step s+2, one row per slot, and with the
                // first row the scale data
                const int r8 = (m - 17) / 3;
                const int64_t j0 = min(s + 2, steps - 1) * kBK;
                pl.c[r8] = __builtin_amdgcn_raw_buffer_load_b32(c_rs, c_off[r8], (int)(j0 * (K / 2)), 0);
                if (r8 == 0) load_scale(j0, pl);
            }
            // patch of step s+1
            if (m >= kLookAhead && m - kLookAhead < 32) {
                const int u = m - kLookAhead, r8 = u / 4, hb = u % 4;
                rows[r8][hb] = scale_pair(lq[u % kLookRing], sc[r8]);
            }
            if (m == 0) own = own_scale(pc);
            if (m < 32) {
                const int u = m, r8 = u / 4, hb = u % 4;
                if (hb == 0) sc[r8] = row_scale(own, r8);
                lq[u % kLookRing] = level(pc.c[r8], hb);
            }
            if (m == kPatchWrite) transpose8x8(rows, cols);
            if (m >= kPatchWrite && m < kPatchWrite + 8) {
                const int e = m - kPatchWrite, c = 8 * cp + e;
                *reinterpret_cast<u32x4 *>(wbuf + nxt * kBTile + tile_seg(c) * 128 + 16 * (jp ^ (c & 7))) = cols[e];
            }
            mfma32(acc[i][jt], fa[ks & 1][i], fb[ks & 1][jt]);
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
        const float own = own_scale(pa);
#pragma unroll
        for (int r8 = 0; r8 < 8; ++r8) {
            const float s8 = row_scale(own, r8);
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) rows[r8][hb] = scale_pair(level(pa.c[r8], hb), s8);
        }
        write_patch(rows, 0);
    }
    __syncthreads();  // W tile 0
    // the operands of step 0's first kFragAhead slots (slot m < 8: ks 0)
#pragma unroll
    for (int jt = 0; jt < kTN; ++jt) fb[0][jt] = bfrag(wbuf, 0, jt);
    fa[0][0] = afrag(ybuf, 0, 0);
    fa[0][1] = afrag(ybuf, 0, 1);
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
    // B operand of lane (lr, h), tile jt, substep ks: A[c][k] for the 8
    // consecutive k = 64 sa + 32 h + 8 ks + e (rows of A are contiguous in k).
    if (p.u != nullptr) {
        const Rsrc u_rs = rsrc(p.u + m0 * p.rp, m_rows * p.rp * 2);
        uint32_t u_off[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int row = seg_row(64 * w + 8 * q + (lane >> 3));
            const int chunk = (lane & 7) ^ (row & 7);
            u_off[q] = (uint32_t)(row * p.rp * 2 + chunk * 16);
        }
        for (int64_t sa = 0; sa < p.rp / kBK; ++sa) {
            char *dst = ybuf + (64 * w) * 128;
#pragma unroll
            for (int q = 0; q < 8; ++q)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(u_rs, (lds_void *)(dst + q * 1024), 16, u_off[q],
                                                         (int)(sa * (kBK * 2)), 0, 0);
            u32x4 ba[4][kTN];
#pragma unroll
            for (int jt = 0; jt < kTN; ++jt) {
                const int64_t c = c0 + 128 * wc + 32 * jt + lr;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    const int64_t k = 64 * sa + 32 * h + 8 * ks;
                    u32x4 v = u32x4{0, 0, 0, 0};
                    if (c < K && k < p.r) v = *reinterpret_cast<const u32x4 *>(p.a + c * p.r + k);
                    ba[ks][jt] = v;
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            valu_to_mfma();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int i = 0; i < kTM; ++i) {
                    const u32x4 av = afrag(ybuf, ks, i);
#pragma unroll
                    for (int jt = 0; jt < kTN; ++jt) mfma32(acc[i][jt], av, ba[ks][jt]);
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
        asm volatile("" : "+a"(acc[i][0]), "+a"(acc[i][1]), "+a"(acc[i][2]), "+a"(acc[i][3]));
    __syncthreads();
    {
        // the wave's 128 x 128 bf16 block through LDS: row stride 256 B,
        // 16-byte chunks XOR-swizzled by row, then 16-byte stores along rows.
        // Accumulator v of tile (i, jt): row 32 i + 8 (v / 4) + 4 h + v % 4,
        // column 32 jt + lr.
        char *const ep = smem + w * 32768;
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int j = 0; j < kTN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 32 * i + 8 * (v >> 2) + 4 * h + (v & 3), cc = 32 * j + lr;
                    const int chunk = (cc >> 3) ^ ((row >> 2) & 15);
                    *reinterpret_cast<uint16_t *>(ep + row * 256 + chunk * 16 + (cc & 7) * 2) =
                        (uint16_t)(pack_bf16x2(acc[i][j][v], 0.0f) & 0xFFFFu);
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
