// linear_gemv.hip - decode-shaped fused NF4 linear (M <= 16 activation rows)
// for gfx950: Y[M x N] = X[M x K] . dequantize(W)^T, W stored [N x K] NF4
// ([MF] "Forward Pass Computation"; source key in nf4_internal.h).
//
// The weight is streamed once from HBM and never materialised. X is padded
// to 16 rows and the contraction runs on v_mfma_f32_16x16x32_bf16 with
// A = X rows and B = 16 weight rows (16 output columns); lane l = 16 g + r
// holds row r of both operands.
//
// Streaming. The unit of work is 16 weight rows x 4 blocks: one 128-byte run
// of each row (2 KiB). A lane fetches it with two 16-byte loads, so one load
// instruction covers 64 contiguous bytes of each of 16 rows: lane group g gets
// bytes [16 g, 16 g + 16) of a pair of blocks, i.e. half a block. The MFMA
// needs all four lane groups inside one block (its k-sum is scaled by that
// block's c1' afterwards), so one v_permlane32_swap_b32 per register pair
// exchanges the upper half-wave of one register with the lower half-wave of
// the other: afterwards lane group g holds 16 consecutive weights
// k = 64 b + 16 s(g) + [0, 16) of every block b, with s = (0, 2, 1, 3), and
// the X operand is loaded in the same order. Units stream through a ring of
// registers several units deep, issued before the unit that uses them is
// computed, so a wave always has most of its ring in flight.
//
// Codes become bf16 pairs through a 256-entry table (byte -> (q[lo], q[hi])
// rounded to bf16) held in LDS once per lane: entry e of lane l is the word
// at byte 256 e + 4 l, so a lane always reads its own bank and the
// data-dependent lookups never conflict. One v_perm_b32 builds each address
// (byte k of the code word next to the lane offset).
//
// Work split: a workgroup of kWaves waves owns NT tiles of 16 output columns
// and all of K. K is cut into chunks of 256 (one unit per tile); wave w takes
// chunks w, w + kWaves, ... and keeps one partial tile per column tile in
// registers; the partials are summed through LDS at the end. NT is chosen so
// that the grid is about one workgroup per CU.
#include <algorithm>
#include <utility>

#include "gemm_common.h"

namespace nf4 {
namespace {

using gemm::Rsrc;
using gemm::rsrc;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Cache policy of the m = 1 kernel's loads of data a call reads exactly once
// (the codes and the per-block scale codes): non-temporal (the `nt` bit of
// the buffer instruction's cache-policy operand). On the 28672 x 8192 weight
// a plain read-only walk took about 20 us with ordinary loads against 18 us
// with non-temporal ones, and the m = 1 kernel gained 3-4%. The staged
// kernel's direct-to-LDS code loads ran slower with the bit, so they and the
// generic kernel keep the ordinary policy, as do x and the shared c2 values.
constexpr int kOnce = 2;
constexpr int kBpu = 4;      // blocks per unit (K chunk of 256 weights)
constexpr int kChunk = kBpu * kBlock;
constexpr int kMaxNT = 8;    // column tiles per workgroup
constexpr int kWaves = 8;    // waves per workgroup (the K split)
constexpr int kMaxK = 32768; // longest row: its E4M3 codes for 16 kMaxNT rows fill kQ8Words
// Staging areas filled by direct-to-LDS loads, which write all 64 lanes'
// dwords (zeros past the source), so each is a whole number of 64-dword loads.
constexpr int round64w(int n) { return (n + 63) / 64 * 64; }
constexpr int kQ8Words = round64w(16 * kMaxNT * (kMaxK / kBlock) / 4 + 64);  // staged E4M3 code dwords
constexpr int kC2Words = round64w(16 * kMaxNT * (kMaxK / kBlock) / 256 + 2);  // staged c2 values

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// f(integral_constant<int, J>) for J = 0 .. N-1, unrolled at compile time.
template <class F, int... J>
__device__ __forceinline__ void static_for_seq(F &&f, std::integer_sequence<int, J...>) {
    (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// One unit's operands for this lane: two 16-byte pieces of codes of weight
// row r (blocks 0-1 and 2-3 of the chunk, lane group g's quarter of each
// pair), and without double quantization the fp32 absmax values of the
// row's 4 blocks. With double quantization the scale data of the
// workgroup's rows is staged in LDS once (see gemv_kernel) and read per unit.
template <bool kDQ> struct Unit;
template <> struct Unit<true> {
    u32x4 c[2];
};
template <> struct Unit<false> {
    u32x4 c[2];
    f32x4 am;
};

// Scale data of one unit for this lane's weight row: the 4 E4M3 codes and
// the group's c2, or the 4 fp32 absmax values.
template <bool kDQ> struct Scales;
template <> struct Scales<true> {
    uint32_t q8;
    float c2;
};
template <> struct Scales<false> {
    f32x4 am;
};

// Per-lane constants of the loads. Buffer descriptors start at the
// workgroup's first weight row and end at its last valid one. Everything
// that selects a row is in the per-lane offset, which the descriptor's range
// check covers, so rows past N read as zero codes and zero scales (and are
// never stored); the scalar offset only moves along a row. Loads of units
// past the wave's last one are still issued, so that the wait counts are the
// same on every path, but through `none`, an empty descriptor, so they return
// zeros without touching memory.
struct Stream {
    Rsrc codes, q, x, none;
    uint32_t c_off;    // r * K/2 + 16 g
    uint32_t q_off;    // 4 r * nblk: bytes of absmax before row r (without double quantization)
    uint32_t x_off;    // bytes of X row r at k = 16 s(g)
    uint32_t tile_c;   // 16 * K/2: bytes of codes per 16 rows
    uint32_t tile_b;   // 16 * nblk: blocks per 16 rows
};

template <bool kDQ>
__device__ __forceinline__ void issue_unit(Unit<kDQ> &u, const Stream &st, int t, uint32_t chunk, bool live) {
    const Rsrc cr = live ? st.codes : st.none;
    const uint32_t vo = st.c_off + (uint32_t)t * st.tile_c;
    u.c[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, vo, (int)(128u * chunk), 0));
    u.c[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, vo + 64u, (int)(128u * chunk), 0));
    if constexpr (!kDQ) {
        const uint32_t tb = (uint32_t)t * st.tile_b;  // block of row 16 t + r, block 0, relative to row r
        const Rsrc ar = live ? st.q : st.none;
        u.am = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(ar, st.q_off + 4u * tb, (int)(4u * kBpu * chunk), 0));
    }
}

// X operand of one chunk: for block j, xa = k 64 j + 16 s(g) + [0, 8) and
// xb = the next 8 of row r (zero for r >= m: the descriptor ends at row m).
__device__ __forceinline__ void issue_x(u32x4 (&xa)[kBpu], u32x4 (&xb)[kBpu], const Stream &st, uint32_t chunk,
                                        bool live) {
    const Rsrc xr = live ? st.x : st.none;
    const int so = (int)(2u * kChunk * chunk);
#pragma unroll
    for (int j = 0; j < kBpu; ++j) {
        xa[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, st.x_off + 128u * j, so, 0));
        xb[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, st.x_off + 128u * j + 16u, so, 0));
    }
}

template <bool kDQ, int J>
__device__ __forceinline__ float unit_scale(const Scales<kDQ> &sc) {
    // gfx950's fp8 -> f32 convert decodes OCP E4M3FN exactly
    if constexpr (kDQ) return __builtin_amdgcn_cvt_f32_fp8((int)sc.q8, J) * sc.c2;
    else return sc.am[J];
}

// bf16 pairs of the 4 code bytes of d: table words at byte 256 * byte + lane4.
__device__ __forceinline__ u32x4 lookup4(const char *lds, uint32_t d, uint32_t lane4) {
    u32x4 v;
    v.x = *reinterpret_cast<const uint32_t *>(lds + __builtin_amdgcn_perm(d, lane4, 0x0C0C0400u));
    v.y = *reinterpret_cast<const uint32_t *>(lds + __builtin_amdgcn_perm(d, lane4, 0x0C0C0500u));
    v.z = *reinterpret_cast<const uint32_t *>(lds + __builtin_amdgcn_perm(d, lane4, 0x0C0C0600u));
    v.w = *reinterpret_cast<const uint32_t *>(lds + __builtin_amdgcn_perm(d, lane4, 0x0C0C0700u));
    return v;
}

template <bool kDQ, int J, int kMI>
__device__ __forceinline__ void block_scale(f32x4_t &acc, const Scales<kDQ> &sc, const f32x4_t &p) {
    // D row 4 g + i, column r: that column is weight row n, scaled by c1'(n, b)
    const float s = unit_scale<kDQ, J>(sc);
    if constexpr (kMI == 1) {
        acc[0] += p[0] * s;  // one activation row: only element 0 of lane group 0 is kept
    } else {
        acc += p * s;
    }
}

__device__ __forceinline__ f32x4_t mfma(const u32x4 &x, const u32x4 &w, const f32x4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(x), as_bf16x8(w), c, 0, 0, 0);
}

// One unit: regroup the code words so that each register holds one block
// (the lower half-wave of block 2p's word pair and the upper half-wave of
// block 2p + 1's are exchanged), then 2 MFMAs per block (first half of the
// block's k with a zero accumulator, then the second half), then the
// block's scale. The order is fixed by scheduling barriers so that table
// reads run a block ahead of the MFMAs that use them and the scaling waits
// on MFMA results that have had time to complete.
template <bool kDQ, int kMI>
__device__ __forceinline__ void unit_mac(f32x4_t &acc, const Unit<kDQ> &u, const Scales<kDQ> &sc,
                                         const u32x4 (&xa)[kBpu], const u32x4 (&xb)[kBpu], const char *lds,
                                         uint32_t lane4) {
    uint32_t ev[kBpu], od[kBpu];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const auto e = __builtin_amdgcn_permlane32_swap(u.c[p].x, u.c[p].z, false, false);
        const auto o = __builtin_amdgcn_permlane32_swap(u.c[p].y, u.c[p].w, false, false);
        ev[2 * p] = e[0];
        ev[2 * p + 1] = e[1];
        od[2 * p] = o[0];
        od[2 * p + 1] = o[1];
    }
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    u32x4 lo[kBpu], hi[kBpu];
    f32x4_t p[kBpu];
    lo[0] = lookup4(lds, ev[0], lane4);
    lo[1] = lookup4(lds, ev[1], lane4);
    hi[0] = lookup4(lds, od[0], lane4);
    hi[1] = lookup4(lds, od[1], lane4);
    __builtin_amdgcn_sched_barrier(0);
    p[0] = mfma(xa[0], lo[0], z);
    p[1] = mfma(xa[1], lo[1], z);
    __builtin_amdgcn_sched_barrier(0);
    lo[2] = lookup4(lds, ev[2], lane4);
    lo[3] = lookup4(lds, ev[3], lane4);
    __builtin_amdgcn_sched_barrier(0);
    p[0] = mfma(xb[0], hi[0], p[0]);
    p[1] = mfma(xb[1], hi[1], p[1]);
    __builtin_amdgcn_sched_barrier(0);
    hi[2] = lookup4(lds, od[2], lane4);
    hi[3] = lookup4(lds, od[3], lane4);
    __builtin_amdgcn_sched_barrier(0);
    p[2] = mfma(xa[2], lo[2], z);
    p[3] = mfma(xa[3], lo[3], z);
    __builtin_amdgcn_sched_barrier(0);
    block_scale<kDQ, 0, kMI>(acc, sc, p[0]);
    block_scale<kDQ, 1, kMI>(acc, sc, p[1]);
    __builtin_amdgcn_sched_barrier(0);
    p[2] = mfma(xb[2], hi[2], p[2]);
    p[3] = mfma(xb[3], hi[3], p[3]);
    __builtin_amdgcn_sched_barrier(0);
    block_scale<kDQ, 2, kMI>(acc, sc, p[2]);
    block_scale<kDQ, 3, kMI>(acc, sc, p[3]);
}

template <int NT, bool kDQ, int kMI>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(const uint16_t *__restrict__ x, int m, WView w,
                                                           uint16_t *__restrict__ y, Levels lv) {
    // Ring of kRing units per wave; chunk i's X goes to buffer i % kNX. With
    // at least 4 tiles the ring is one chunk's tiles (kR = 1); with fewer it
    // spans two chunks. The issue of chunk i + 1's first unit must not
    // overwrite an X buffer still in use, hence kNX = kR + 1 buffers, and the
    // loop is unrolled over kUnroll units so that every ring slot, X buffer
    // and accumulator index is a compile-time constant.
    constexpr int kR = NT >= 4 ? 1 : 2;
    constexpr int kRing = kR * NT;
    constexpr int kNX = kR + 1;
    constexpr int kUnroll = NT * (kR == 1 ? 2 : 6);
    // vector-memory loads of the prologue (units 0 .. kRing - 2 and the X of
    // the chunks they start)
    constexpr int kPrologueLoads = (kRing - 1) * (kDQ ? 2 : 3) + 2 * kBpu * ((kRing - 2) / NT + 1);
    static_assert(kPrologueLoads < 64, "vmcnt range");
    static_assert(kUnroll % kRing == 0 && (kUnroll / NT) % kNX == 0, "unroll must align ring and X buffers");
    static_assert(kWaves * NT * 256 <= 256 * 64, "partial tiles must fit the table's LDS");

    // 64 KiB: the lane-replicated code table, then the partial tiles
    __shared__ uint32_t s_lds[256 * 64];
    __shared__ float s_lv[16];
    // with double quantization: the E4M3 codes of the workgroup's rows (row
    // rho's dword d at rho * K/256 + (d ^ (rho & qmask))) and the c2 values
    // of its groups
    __shared__ uint32_t s_q8[kDQ ? kQ8Words : 1];
    __shared__ float s_c2[kDQ ? kC2Words : 1];
    const char *lds = reinterpret_cast<const char *>(s_lds);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int sg = ((g & 1) << 1) | (g >> 1);  // the block quarter lane group g ends up with
    const uint32_t lane4 = 4u * lane;
    const int64_t K = w.k, nblk = K / kBlock;
    const int64_t n_base = (int64_t)blockIdx.x * 16 * NT;
    const int64_t rows = std::min<int64_t>(w.n - n_base, 16 * NT);

    Stream st;
    st.tile_c = (uint32_t)(16 * (K / 2));
    st.tile_b = (uint32_t)(16 * nblk);
    st.none = rsrc(w.codes, 0);
    st.codes = rsrc(w.codes + n_base * (K / 2), rows * (K / 2));
    st.x = rsrc(x, (int64_t)m * K * 2);
    st.c_off = (uint32_t)(r * (K / 2) + 16 * g);
    st.x_off = (uint32_t)(2 * (r * K + 16 * sg));

    // Scale data. With double quantization the workgroup's E4M3 codes (rows
    // x K/64 bytes, contiguous in memory) and its groups' c2 values are
    // copied to LDS by direct-to-LDS loads issued before anything else, so
    // every scale line is fetched once per workgroup instead of once per unit.
    // A row's dwords are XOR-swizzled by the row index (within aligned runs of
    // up to 32 dwords) so that the 16 rows a unit reads fall in distinct banks.
    const uint32_t rowdw = (uint32_t)(nblk / 4);  // E4M3 code dwords per row
    const uint32_t qmask = std::min(rowdw & (0u - rowdw), 32u) - 1u;
    uint32_t c2_row0 = 0;  // block index of row n_base + r, block 0, counted from the first staged group
    if constexpr (kDQ) {
        const int64_t g0 = n_base * nblk / 256, g1 = ((n_base + rows) * nblk - 1) / 256;
        c2_row0 = (uint32_t)((n_base + r) * nblk - g0 * 256);
        const Rsrc qsrc = rsrc(w.q + n_base * nblk, rows * nblk);
        const uint32_t total = (uint32_t)rows * rowdw;
        constexpr uint32_t kStep = 64u * kWaves;
        uint32_t rho = (uint32_t)(wave * 64 + lane) / rowdw;
        uint32_t d = (uint32_t)(wave * 64 + lane) - rho * rowdw;
        const uint32_t sq = kStep / rowdw, sr = kStep - sq * rowdw;
        for (uint32_t p0 = (uint32_t)wave * 64u; p0 < total; p0 += kStep) {
            // dwords p0 + lane of the staged array; past `total` the source is
            // outside the descriptor and zeros are written (inside s_q8)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(qsrc, (gemm::lds_void *)(s_q8 + p0), 4,
                                                     (rho * rowdw + (d ^ (rho & qmask))) * 4u, 0, 0, 0);
            rho += sq;
            d += sr;
            if (d >= rowdw) {
                d -= rowdw;
                ++rho;
            }
        }
        const Rsrc csrc = rsrc(w.scale + g0, (g1 - g0 + 1) * 4);
        for (uint32_t p0 = (uint32_t)wave * 64u; p0 < (uint32_t)(g1 - g0 + 1); p0 += kStep)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(csrc, (gemm::lds_void *)(s_c2 + p0), 4, (p0 + lane) * 4u, 0,
                                                     0, 0);
    } else {
        st.q = rsrc(w.absmax + n_base * nblk, rows * nblk * 4);
        st.q_off = (uint32_t)(r * nblk * 4);
    }

    // this wave's chunks: wave, wave + kWaves, ...; unit u = (chunk u / NT, tile u % NT)
    const int64_t chunks = K / kChunk;
    const int nc = wave < chunks ? (int)((chunks - wave + kWaves - 1) / kWaves) : 0;
    const int units = nc * NT;

    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    Unit<kDQ> ring[kRing];
    u32x4 xa[kNX][kBpu], xb[kNX][kBpu];

    // Issue unit u (u0 + UJ with u0 a multiple of kUnroll): its chunk's X first
    // when it is the chunk's first tile. Issued whether or not the unit exists.
    auto issue = [&](int u0, auto UJ) {
        constexpr int J = decltype(UJ)::value;
        constexpr int t = J % NT, ci = J / NT;
        const int u = u0 + J;
        const bool live = u < units;
        const uint32_t chunk = (uint32_t)(wave + kWaves * (u / NT));
        if constexpr (t == 0) issue_x(xa[ci % kNX], xb[ci % kNX], st, chunk, live);
        issue_unit<kDQ>(ring[J % kRing], st, t, chunk, live);
    };

    // prologue: the first kRing - 1 units, issued before the table is built
    static_for<kRing - 1>([&](auto JC) { issue(0, JC); });

    // The levels arrive as kernel arguments (scalar loads); a select chain
    // writes them to LDS so that the table is built without vector-memory
    // loads, which would wait for the units issued above.
    if (tid < 16) {
        // (the empty asm keeps each level an opaque scalar, so the chain is
        // not turned back into an indexed load of the argument block)
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float q = lv.q[i];
            asm volatile("" : "+s"(q));
            v = tid == i ? q : v;
        }
        s_lv[tid] = v;
    }
    __syncthreads();
    for (int i = tid; i < 256 * 64; i += 64 * kWaves) {
        const int e = i >> 6;
        s_lds[i] = pack_bf16x2(s_lv[e & 15], s_lv[e >> 4]);
    }
    // this wave's scale copies have landed once at most the prologue's
    // vector-memory loads (issued after them) are outstanding; the barrier
    // then publishes every wave's copies
    if constexpr (kDQ) __builtin_amdgcn_s_waitcnt(gemm::vmcnt_at_most(kPrologueLoads));
    __syncthreads();

    for (int u0 = 0; u0 < units; u0 += kUnroll) {
        static_for<kUnroll>([&](auto JC) {
            constexpr int J = decltype(JC)::value;
            constexpr int t = J % NT, ci = J / NT;
            // keep kRing - 1 units in flight ahead of this one
            if constexpr (J + kRing - 1 < kUnroll) {
                issue(u0, std::integral_constant<int, J + kRing - 1>{});
            } else {
                issue(u0 + kUnroll, std::integral_constant<int, J + kRing - 1 - kUnroll>{});
            }
            if (u0 + J < units) {
                Scales<kDQ> sc;
                if constexpr (kDQ) {
                    const uint32_t chunk = (uint32_t)(wave + kWaves * ((u0 + J) / NT));
                    const uint32_t row = 16u * t + r;
                    sc.q8 = s_q8[row * rowdw + (chunk ^ (row & qmask))];
                    sc.c2 = s_c2[(c2_row0 + (uint32_t)t * st.tile_b + kBpu * chunk) >> 8];
                } else {
                    sc.am = ring[J % kRing].am;
                }
                unit_mac<kDQ, kMI>(acc[t], ring[J % kRing], sc, xa[ci % kNX], xb[ci % kNX], lds, lane4);
            }
        });
    }

    // Sum the waves' partial tiles through LDS: [tile][i][wave][lane] floats.
    __syncthreads();
    float *red = reinterpret_cast<float *>(s_lds);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < kMI; ++i) red[((t * 4 + i) * kWaves + wave) * 64 + lane] = acc[t][i];
    __syncthreads();
    for (int e = tid; e < NT * 256; e += 64 * kWaves) {
        const int t = e >> 8, i = (e >> 6) & 3, l = e & 63;
        const int row = 4 * (l >> 4) + i;
        const int64_t n = n_base + 16 * t + (l & 15);
        if (i < kMI && row < m && n < w.n) {
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < kWaves; ++v) s += red[((t * 4 + i) * kWaves + v) * 64 + l];
            y[(int64_t)row * w.n + n] = (uint16_t)(pack_bf16x2(s, 0.0f) & 0xFFFFu);
        }
    }
}

// ---- one activation row (m == 1): VALU dot products over row-linear loads
//
// With a single activation row the MFMA's 16-row A operand is 1/16 used and
// the 16-row tile makes every load touch 16 weight rows. Here one wave
// handles one weight row at a time and streams its codes linearly, 1 KiB per
// load instruction: in piece p of a row, lane l holds the 16 code bytes of
// weights k = 2048 p + 32 l + [0, 32), one half of block 32 p + l/2. Wave g
// of the W waves of the grid takes rows g, g + W, g + 2W, ..., so at any
// moment the whole chip reads one window of consecutive rows: HBM streams
// such a sweep faster than the same bytes read as one contiguous region per
// wave. Code bytes become bf16 level pairs through the lane-private table,
// v_dot2c_f32_bf16 multiplies them with the lane's x pairs, and the
// half-block sum is scaled by its c1' (one FMA). At the end of a row a wave
// reduction adds the 64 lanes and lane 0 stores y. Requires K = P * 2048
// with P <= 4. With double quantization a row's E4M3 codes (32 P bytes)
// arrive with its first piece, one dword per lane, and each piece takes its
// lanes' codes from there with one ds_bpermute; the row's c2 is one value, as
// K is a divisor of 256 x 64 weights.
//
// x sits in LDS beside the table (up to 16 KiB) and each piece reads its
// lane's 64 bytes of it: held in registers for the whole kernel it took 64
// VGPRs per lane and capped the CU at 16 waves. With x in LDS a wave needs
// about 80 VGPRs, and two 12-wave workgroups (the table plus x fill the
// 160 KiB of LDS) keep 24 waves, so 72 rather than 48 pieces in flight per
// CU.
constexpr int kWaves1 = 12;
constexpr int kRing1 = 4;      // pieces in flight per wave
constexpr int kPiece = 2048;   // weights per piece: one 1 KiB load instruction
constexpr int kMaxP1 = 4;      // pieces per row (x in LDS: 4 KiB per piece)

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <bool kDQ> struct Piece;
template <> struct Piece<true> {
    u32x4 c;
    uint32_t q8w;  // first piece of a row: E4M3 codes of blocks 4 (lane % 8P) .. + 3
    float c2;      // first piece of a row: the row's c2
};
template <> struct Piece<false> {
    u32x4 c;
    float am;
};

// Sum over the 64 lanes (every lane gets the sum).
__device__ __forceinline__ float wave_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(h[0]) + __uint_as_float(h[1]);  // rows 0+1 and 2+3
    const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// LDS byte offset of chunk i (x pairs 4i .. 4i+3) of lane l's part of piece
// p: 4096 p + 64 l + 16 ((i + l / 4) % 4). The rotation puts the 16 lanes of
// an aligned group, reading one chunk index, on 16 distinct 16-byte bank
// groups.
__device__ __forceinline__ uint32_t x_slot(int p, int l, int i) {
    return (uint32_t)(4096 * p + 64 * l + 16 * ((i + (l >> 2)) & 3));
}

template <int P, bool kDQ>
__global__ __launch_bounds__(64 * kWaves1) __attribute__((amdgpu_waves_per_eu(6))) void gemv1_kernel(
    const uint16_t *__restrict__ x, WView w, uint16_t *__restrict__ y, Levels lv) {
    static_assert(kRing1 % P == 0, "ring must hold whole rows' pieces in phase");
    constexpr int kXChunks = P * 256;  // 16-byte chunks of x
    constexpr int kXIters = (kXChunks + 64 * kWaves1 - 1) / (64 * kWaves1);
    __shared__ uint32_t s_lds[256 * 64];
    __shared__ __align__(16) char s_x[P * 4096];
    const char *lds = reinterpret_cast<const char *>(s_lds);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lane4 = 4u * lane;
    const int64_t K = w.k, nblk = K / kBlock;
    const int64_t W = (int64_t)gridDim.x * kWaves1, gw = (int64_t)blockIdx.x * kWaves1 + wave;
    // this wave's rows: gw, gw + W, gw + 2W, ...
    const int nrows = gw < w.n ? (int)((w.n - 1 - gw) / W + 1) : 0;
    const int npieces = nrows * P;

    // one descriptor per row (no offset grows with the matrix); loads of
    // pieces past the end go through an empty descriptor (the wait counts
    // then match on every path)
    const Rsrc none = rsrc(w.codes, 0);
    const uint32_t half_blk = (uint32_t)(lane >> 1);  // lane's block within a piece

    Piece<kDQ> ring[kRing1];
    auto issue = [&](int j0, auto JC) {
        constexpr int J = decltype(JC)::value;
        constexpr int pp = J % P;
        const int j = j0 + J;
        const bool live = j < npieces;
        const int64_t row = gw + (int64_t)(j0 / P + J / P) * W;
        Piece<kDQ> &pc = ring[J % kRing1];
        const Rsrc cr = live ? rsrc(w.codes + row * (K / 2), K / 2) : none;
        pc.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(cr, 16u * lane, 1024 * pp, kOnce));
        if constexpr (kDQ) {
            if constexpr (pp == 0) {
                const Rsrc qr = live ? rsrc(w.q + row * nblk, nblk) : none;
                pc.q8w = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(qr, 4u * (uint32_t)(lane & (8 * P - 1)), 0, kOnce);
                const Rsrc sr = live ? rsrc(w.scale + ((row * nblk) >> 8), 4) : none;
                pc.c2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 0u, 0, 0));
            }
        } else {
            const Rsrc ar = live ? rsrc(w.absmax + row * nblk, nblk * 4) : none;
            pc.am = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ar, 4u * (32u * pp + half_blk), 0, kOnce));
        }
    };

    static_for<kRing1 - 1>([&](auto JC) { issue(0, JC); });

    // x: chunk c (bytes 16 c .. 16 c + 15) is chunk c % 4 of lane (c / 4) % 64
    // of piece c / 256
    u32x4 xc[kXIters];
    {
        const Rsrc xr = rsrc(x, K * 2);
#pragma unroll
        for (int j = 0; j < kXIters; ++j) {
            const int c = tid + 64 * kWaves1 * j;
            if (c < kXChunks) xc[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, 16u * c, 0, 0));
        }
    }

    // the 16 levels go through the x area first (the empty asm keeps each an
    // opaque scalar, so the chain is not turned back into an indexed load of
    // the argument block); the table is built from there, then x replaces them
    float *const s_lv = reinterpret_cast<float *>(s_x);
    if (tid < 16) {
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float q = lv.q[i];
            asm volatile("" : "+s"(q));
            v = tid == i ? q : v;
        }
        s_lv[tid] = v;
    }
    __syncthreads();
    for (int i = tid; i < 256 * 64; i += 64 * kWaves1) {
        const int e = i >> 6;
        s_lds[i] = pack_bf16x2(s_lv[e & 15], s_lv[e >> 4]);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kXIters; ++j) {
        const int c = tid + 64 * kWaves1 * j;
        if (c < kXChunks)
            *reinterpret_cast<u32x4 *>(s_x + x_slot(c >> 8, (c >> 2) & 63, c & 3)) = xc[j];
    }
    __syncthreads();
    uint32_t xo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xo[i] = x_slot(0, lane, i);

    float acc = 0.0f;
    uint32_t row_q8w = 0;  // the current row's scale data, kept past its ring slot
    float row_c2 = 0.0f;
    for (int j0 = 0; j0 < npieces; j0 += kRing1) {
        static_for<kRing1>([&](auto JC) {
            constexpr int J = decltype(JC)::value;
            constexpr int pp = J % P;
            if constexpr (J + kRing1 - 1 < kRing1) {
                issue(j0, std::integral_constant<int, J + kRing1 - 1>{});
            } else {
                issue(j0 + kRing1, std::integral_constant<int, J - 1>{});
            }
            if (j0 + J < npieces) {
                const Piece<kDQ> &pc = ring[J % kRing1];
                // the level-pair lookups and the scale first, then the dot
                // products on two chains
                float sc;
                if constexpr (kDQ) {
                    if constexpr (pp == 0) {
                        row_q8w = pc.q8w;
                        row_c2 = pc.c2;
                    }
                    // block 32 pp + lane/2 sits in byte (lane/2) % 4 of lane 8 pp + lane/8's dword
                    const uint32_t dw = (uint32_t)__builtin_amdgcn_ds_bpermute(
                        (int)(4u * (8u * pp + (uint32_t)(lane >> 3))), (int)row_q8w);
                    sc = __builtin_amdgcn_cvt_f32_fp8((int)(dw >> (8u * (half_blk & 3u))), 0) * row_c2;
                } else {
                    sc = pc.am;
                }
                u32x4 xv[4], lv4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = *reinterpret_cast<const u32x4 *>(s_x + 4096 * pp + xo[i]);
#pragma unroll
                for (int i = 0; i < 4; ++i) lv4[i] = lookup4(lds, pc.c[i], lane4);
                __builtin_amdgcn_sched_barrier(0);
                float part[2] = {0.0f, 0.0f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // (vector elements are copied to scalars first: a bit cast of
                        // an element expression reads element 0 with this compiler)
                        const uint32_t lw = lv4[i][b], xw = xv[i][b];
                        part[b & 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, lw),
                                                                      __builtin_bit_cast(bf16x2_t, xw), part[b & 1],
                                                                      false);
                    }
                }
                acc = fmaf(part[0] + part[1], sc, acc);
                if constexpr (pp == P - 1) {
                    const float sum = wave_sum(acc);
                    const int64_t row = gw + (int64_t)(j0 / P + J / P) * W;
                    if (lane == 0) y[row] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xFFFFu);
                    acc = 0.0f;
                }
            }
        });
    }
}

template <bool kDQ>
void launch_gemv1(int p, dim3 grid, const uint16_t *x, const WView &w, uint16_t *y, hipStream_t s) {
    switch (p) {
        case 1: gemv1_kernel<1, kDQ><<<grid, dim3(64 * kWaves1), 0, s>>>(x, w, y, levels()); break;
        case 2: gemv1_kernel<2, kDQ><<<grid, dim3(64 * kWaves1), 0, s>>>(x, w, y, levels()); break;
        default: gemv1_kernel<4, kDQ><<<grid, dim3(64 * kWaves1), 0, s>>>(x, w, y, levels()); break;
    }
}

template <int NT, int kMI>
void launch_nt(dim3 grid, const uint16_t *x, int m, const WView &w, uint16_t *y, hipStream_t s) {
    if (w.q)
        gemv_kernel<NT, true, kMI><<<grid, dim3(64 * kWaves), 0, s>>>(x, m, w, y, levels());
    else
        gemv_kernel<NT, false, kMI><<<grid, dim3(64 * kWaves), 0, s>>>(x, m, w, y, levels());
}

template <int kMI>
void launch_mi(int nt, dim3 grid, const uint16_t *x, int m, const WView &w, uint16_t *y, hipStream_t s) {
    switch (nt) {
        case 1: launch_nt<1, kMI>(grid, x, m, w, y, s); break;
        case 2: launch_nt<2, kMI>(grid, x, m, w, y, s); break;
        case 3: launch_nt<3, kMI>(grid, x, m, w, y, s); break;
        case 4: launch_nt<4, kMI>(grid, x, m, w, y, s); break;
        case 5: launch_nt<5, kMI>(grid, x, m, w, y, s); break;
        case 6: launch_nt<6, kMI>(grid, x, m, w, y, s); break;
        case 7: launch_nt<7, kMI>(grid, x, m, w, y, s); break;
        default: launch_nt<8, kMI>(grid, x, m, w, y, s); break;
    }
}

// ---- 2 <= m <= 16 with K = 2048 QS (QS = 1, 2, 4): long code runs through LDS
//
// The kernel above reads, per load instruction, 64 bytes from each of 16
// weight rows, which streams HBM well below the rate of long contiguous
// runs. Here every code load is one row's contiguous 1 KiB, copied straight
// into LDS (direct-to-LDS), and the 16-row MFMA operands are read from there.
//
// A workgroup of 8 waves owns NT tiles of 16 weight rows and walks them in
// stages: stage s holds tile s / QS, k-range (s % QS) 2048 + [0, 2048) of
// its 16 rows (16 KiB of codes); wave w loads two of the rows and computes
// blocks 4w .. 4w + 3 of every stage for all 16 rows, so each wave's k-ranges
// are fixed and their x stays in registers for the whole kernel. Four stage
// buffers rotate: a stage's loads are issued three stages before it is
// computed, and one barrier per stage both publishes its codes and frees the
// buffer of the stage before. In LDS, 16-byte piece p of stage row r sits at
// slot p ^ r (each lane of a row load fetches piece lane ^ r), so that the
// 16 rows' reads of one block hit distinct banks. The block scales travel in
// a register ring beside the stages. At the end of a tile each wave writes
// its partial 16 x 16 tile to LDS (two buffers, alternating by tile), and
// after the next barrier 256 threads add the 8 waves' partials and store y.
constexpr int kSW = 8;              // waves per workgroup
constexpr int kSR = 4;              // stage buffers
constexpr int kStage = 16 * 1024;   // bytes of codes per stage: 16 rows x 1 KiB

template <bool kDQ> struct StageScales;
template <> struct StageScales<true> {
    uint32_t q8;  // E4M3 codes of the lane's row, its wave's 4 blocks
    float c2;
};
template <> struct StageScales<false> {
    f32x4 am;
};

template <int QS, bool kDQ>
__global__ __launch_bounds__(64 * kSW) void gemv_staged_kernel(const uint16_t *__restrict__ x, int m, WView w,
                                                                uint16_t *__restrict__ y, Levels lv, int nt) {
    constexpr int kOps = 2 + (kDQ ? 2 : 1);  // vector-memory instructions per stage and wave
    static_assert(kSR % QS == 0, "a ring turn holds whole tiles");
    __shared__ uint32_t s_tab[256 * 64];                 // lane-private code -> bf16 pair table
    // the stage buffers as separate arrays, so that the compiler's wait
    // before an LDS read covers only the direct-to-LDS loads into that buffer
    __shared__ __align__(16) char s_stage0[kStage];
    __shared__ __align__(16) char s_stage1[kStage];
    __shared__ __align__(16) char s_stage2[kStage];
    __shared__ __align__(16) char s_stage3[kStage];
    static_assert(kSR == 4, "four stage arrays");
    __shared__ __align__(16) f32x4_t s_part[2][kSW * 64];
    auto stage_buf = [&](auto SLOT) -> char * {
        constexpr int slot = decltype(SLOT)::value;
        if constexpr (slot == 0) return s_stage0;
        else if constexpr (slot == 1) return s_stage1;
        else if constexpr (slot == 2) return s_stage2;
        else return s_stage3;
    };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int64_t K = w.k, nblk = K / kBlock;
    const uint32_t half_k = (uint32_t)(K / 2);
    const int64_t n_base = (int64_t)blockIdx.x * 16 * nt;
    const int64_t rows = std::min<int64_t>(w.n - n_base, 16 * (int64_t)nt);
    const int stages = nt * QS;

    const Rsrc none = rsrc(w.codes, 0);
    const Rsrc cr = rsrc(w.codes + n_base * (K / 2), rows * (K / 2));
    const Rsrc xr = rsrc(x, (int64_t)m * K * 2);
    Rsrc qr, sr;
    if constexpr (kDQ) {
        qr = rsrc(w.q + n_base * nblk, rows * nblk);
        sr = rsrc(w.scale, ((w.n * nblk + 255) / 256) * 4);
    } else {
        qr = rsrc(w.absmax + n_base * nblk, rows * nblk * 4);
        sr = none;
    }

    // x of the wave's blocks: stage position q, block j -> k = 2048 q + 64 (4 wave + j) + 16 g + [0, 16)
    u32x4 xa[QS][4], xb[QS][4];
#pragma unroll
    for (int q = 0; q < QS; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t vo = 2u * (uint32_t)(r * K + 2048 * q + 64 * (4 * wave + j) + 16 * g);
            xa[q][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo, 0, 0));
            xb[q][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, vo + 16u, 0, 0));
        }

    // Stage s's loads: this wave's two rows of codes into buffer s % kSR, and
    // the block scales of the lane's row into ring slot s % kSR. Stages past
    // the last go through the empty descriptor (zeros, no memory traffic), so
    // every stage issues the same instructions.
    StageScales<kDQ> ring[kSR];
    const uint32_t piece = 16u * (uint32_t)lane;
    auto issue = [&](int s, auto SLOT) {
        constexpr int slot = decltype(SLOT)::value;
        const bool live = s < stages;
        const int t = s / QS, q = s % QS;
        char *buf = stage_buf(SLOT);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int rho = 2 * wave + h;
            const uint32_t vo = (uint32_t)(16 * t + rho) * half_k + (piece ^ (16u * (uint32_t)rho));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? cr : none, (gemm::lds_void *)(buf + rho * 1024), 16, vo,
                                                     1024 * q, 0, 0);
        }
        const uint32_t blk = (uint32_t)(16 * t + r) * (uint32_t)nblk + 32u * q + 4u * wave;
        if constexpr (kDQ) {
            ring[slot].q8 = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(live ? qr : none, blk, 0, 0);
            const uint32_t grp = (uint32_t)((n_base * nblk + blk) >> 8);
            ring[slot].c2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(live ? sr : none, 4u * grp, 0, 0));
        } else {
            ring[slot].am = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(live ? qr : none, 4u * blk, 0, 0));
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    __builtin_amdgcn_sched_barrier(0);
    static_for<kSR - 1>([&](auto JC) { issue(decltype(JC)::value, JC); });

    // The table: word i = e * 64 + lane holds (level[e & 15], level[e >> 4])
    // as bf16; thread tid writes i = tid + 512 j, entry e = wave + 8 j.
    {
        const float lo0 = lv.q[wave], lo1 = lv.q[wave + 8];
#pragma unroll
        for (int j = 0; j < 32; ++j) s_tab[tid + 512 * j] = pack_bf16x2((j & 1) ? lo1 : lo0, lv.q[j >> 1]);
    }

    // fragment offsets of the wave's 4 blocks inside a stage (the same in every stage)
    uint32_t foff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        foff[j] = (uint32_t)(r * 1024 + 8 * (g & 1)) + 16u * ((uint32_t)(2 * (4 * wave + j) + (g >> 1)) ^ (uint32_t)r);
    const char *tab = reinterpret_cast<const char *>(s_tab);
    const uint32_t lane4 = 4u * lane;
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t acc = z;

    // 256 threads: the sum of the 8 waves' partials of tile t (from buffer t % 2)
    auto reduce = [&](int t) {
        if (tid < 256) {
            const int i = tid >> 6, l = tid & 63;
            const int row = 4 * (l >> 4) + i;
            const int64_t n = n_base + 16 * t + (l & 15);
            const float *pp = reinterpret_cast<const float *>(s_part[t & 1]);
            float v = 0.0f;
#pragma unroll
            for (int u = 0; u < kSW; ++u) v += pp[(u * 64 + l) * 4 + i];
            if (row < m && n < w.n) y[(int64_t)row * w.n + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
        }
    };

    // (a do-while: stages >= 1, and no branch ahead of the loop that would
    // let the compiler sink the x loads below the prologue's stage loads)
    int s0 = 0;
    do {
        static_for<kSR>([&](auto PC) {
            constexpr int p = decltype(PC)::value;
            constexpr int q = p % QS;
            const int s = s0 + p;
            // this wave's loads of stage s have landed once at most the two
            // stages issued after it are outstanding; the barrier then makes
            // every wave's rows visible and frees the buffer of stage s - 1.
            // A plain s_barrier: the fence of __syncthreads would also wait
            // for the loads of the stages still in flight.
            __builtin_amdgcn_s_waitcnt(gemm::vmcnt_at_most_lds_done(2 * kOps));
            __builtin_amdgcn_s_barrier();
            if (q == 0 && s > 0 && s < stages) reduce(s / QS - 1);
            issue(s + kSR - 1, std::integral_constant<int, (p + kSR - 1) % kSR>{});
            if (s < stages) {
                const char *buf = stage_buf(PC);
                const StageScales<kDQ> &sc = ring[p];
                static_for<4>([&](auto JC) {
                    constexpr int j = decltype(JC)::value;
                    const gemm::u32x2 d = *reinterpret_cast<const gemm::u32x2 *>(buf + foff[j]);
                    const u32x4 lo = lookup4(tab, d.x, lane4);
                    const u32x4 hi = lookup4(tab, d.y, lane4);
                    f32x4_t pr = mfma(xa[q][j], lo, z);
                    pr = mfma(xb[q][j], hi, pr);
                    float scj;
                    if constexpr (kDQ) scj = __builtin_amdgcn_cvt_f32_fp8((int)sc.q8, j) * sc.c2;
                    else scj = sc.am[j];
                    acc += pr * scj;
                });
                if (q == QS - 1) {
                    s_part[(s / QS) & 1][wave * 64 + lane] = acc;
                    acc = z;
                }
            }
        });
        s0 += kSR;
    } while (s0 < stages);
    __builtin_amdgcn_s_waitcnt(gemm::vmcnt_at_most(0));
    __syncthreads();
    reduce(nt - 1);
}

template <int QS, bool kDQ>
void launch_staged(dim3 grid, const uint16_t *x, int m, const WView &w, uint16_t *y, int nt, hipStream_t s) {
    gemv_staged_kernel<QS, kDQ><<<grid, dim3(64 * kSW), 0, s>>>(x, m, w, y, levels(), nt);
}

}  // namespace

// K at most kMaxK: the staged scale data of a workgroup's rows fits LDS.
bool gemv_supported(int64_t m, int64_t k) { return m >= 1 && m <= 16 && k % kChunk == 0 && k <= kMaxK; }

hipError_t launch_gemv(const uint16_t *x, int64_t m, const nf4_weight &wt, uint16_t *y, hipStream_t s) {
    const WView w = make_view(wt);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (m == 1 && w.k % kPiece == 0 && w.k / kPiece <= kMaxP1 && w.k / kPiece != 3) {
        // two workgroups per CU (fewer for a short matrix), the rows dealt
        // round-robin over their waves; the grid is trimmed so that every
        // wave takes the same number of rows, give or take the last one
        const int p = (int)(w.k / kPiece);
        const int64_t rows_per_wave = (w.n + 2 * cus * kWaves1 - 1) / (2 * cus * kWaves1);
        const int64_t g1n = std::min<int64_t>(2 * cus, ((w.n + rows_per_wave - 1) / rows_per_wave + kWaves1 - 1) / kWaves1);
        const dim3 grid1((unsigned)std::max<int64_t>(1, g1n));
        if (w.q)
            launch_gemv1<true>(p, grid1, x, w, y, s);
        else
            launch_gemv1<false>(p, grid1, x, w, y, s);
        return hipGetLastError();
    }
    const int64_t tiles = (w.n + 15) / 16;
    if (m >= 2 && (w.k == 2048 || w.k == 4096 || w.k == 8192)) {
        // stage walk: about one workgroup per CU, each with ceil(tiles / CUs) tiles
        const int nt = (int)std::max<int64_t>((tiles + cus - 1) / cus, 1);
        const dim3 grid((unsigned)((tiles + nt - 1) / nt));
        const int xm = (int)m;
        if (w.k == 8192) w.q ? launch_staged<4, true>(grid, x, xm, w, y, nt, s) : launch_staged<4, false>(grid, x, xm, w, y, nt, s);
        else if (w.k == 4096) w.q ? launch_staged<2, true>(grid, x, xm, w, y, nt, s) : launch_staged<2, false>(grid, x, xm, w, y, nt, s);
        else w.q ? launch_staged<1, true>(grid, x, xm, w, y, nt, s) : launch_staged<1, false>(grid, x, xm, w, y, nt, s);
        return hipGetLastError();
    }
    const int nt = (int)std::min<int64_t>(std::max<int64_t>((tiles + cus - 1) / cus, 1), kMaxNT);
    const dim3 grid((unsigned)((tiles + nt - 1) / nt));
    if (m == 1)
        launch_mi<1>(nt, grid, x, (int)m, w, y, s);
    else
        launch_mi<4>(nt, grid, x, (int)m, w, y, s);
    return hipGetLastError();
}

}  // namespace nf4
