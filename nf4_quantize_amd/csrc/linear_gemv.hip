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

constexpr int kBpu = 4;      // blocks per unit (K chunk of 256 weights)
constexpr int kChunk = kBpu * kBlock;
constexpr int kMaxNT = 8;    // column tiles per workgroup
constexpr int kWaves = 8;    // waves per workgroup (the K split)

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
// pair) and the raw scale data of the row's 4 blocks: the E4M3 codes and the
// group's c2 with double quantization, else the fp32 absmax values.
template <bool kDQ> struct Unit;
template <> struct Unit<true> {
    u32x4 c[2];
    uint32_t q8;
    float c2;
};
template <> struct Unit<false> {
    u32x4 c[2];
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
    Rsrc codes, q, sc, x, none;
    uint32_t c_off;    // r * K/2 + 16 g
    uint32_t q_off;    // r * nblk (bytes of E4M3 codes), or 4 r * nblk (absmax bytes)
    uint32_t flat0;    // block index of row n_base + r, block 0, from the group of row n_base
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
    const uint32_t tb = (uint32_t)t * st.tile_b;  // block of row 16 t + r, block 0, relative to row r
    if constexpr (kDQ) {
        // the 4 blocks share one aligned word of E4M3 codes and one group
        const Rsrc qr = live ? st.q : st.none, sr = live ? st.sc : st.none;
        u.q8 = __builtin_amdgcn_raw_buffer_load_b32(qr, st.q_off + tb, (int)(kBpu * chunk), 0);
        const uint32_t grp = (st.flat0 + tb + kBpu * chunk) >> 8;
        u.c2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, grp * 4u, 0, 0));
    } else {
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
__device__ __forceinline__ float unit_scale(const Unit<kDQ> &u) {
    // gfx950's fp8 -> f32 convert decodes OCP E4M3FN exactly
    if constexpr (kDQ) return __builtin_amdgcn_cvt_f32_fp8((int)u.q8, J) * u.c2;
    else return u.am[J];
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
__device__ __forceinline__ void block_mac(f32x4_t &acc, const Unit<kDQ> &u, uint32_t ev, uint32_t od, const u32x4 &xa,
                                          const u32x4 &xb, const char *lds, uint32_t lane4) {
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    const u32x4 lo = lookup4(lds, ev, lane4), hi = lookup4(lds, od, lane4);
    f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(lo), z, 0, 0, 0);
    p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb), as_bf16x8(hi), p, 0, 0, 0);
    // D row 4 g + i, column r: that column is weight row n, scaled by c1'(n, b)
    const float s = unit_scale<kDQ, J>(u);
    if constexpr (kMI == 1) {
        acc[0] += p[0] * s;  // one activation row: only element 0 of lane group 0 is kept
    } else {
        acc += p * s;
    }
}

// One unit: regroup the code words so that each register holds one block
// (the lower half-wave of block 2p's word pair and the upper half-wave of
// block 2p + 1's are exchanged), then 2 MFMAs per block.
template <bool kDQ, int kMI>
__device__ __forceinline__ void unit_mac(f32x4_t &acc, const Unit<kDQ> &u, const u32x4 (&xa)[kBpu],
                                         const u32x4 (&xb)[kBpu], const char *lds, uint32_t lane4) {
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
    block_mac<kDQ, 0, kMI>(acc, u, ev[0], od[0], xa[0], xb[0], lds, lane4);
    block_mac<kDQ, 1, kMI>(acc, u, ev[1], od[1], xa[1], xb[1], lds, lane4);
    block_mac<kDQ, 2, kMI>(acc, u, ev[2], od[2], xa[2], xb[2], lds, lane4);
    block_mac<kDQ, 3, kMI>(acc, u, ev[3], od[3], xa[3], xb[3], lds, lane4);
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
    static_assert(kUnroll % kRing == 0 && (kUnroll / NT) % kNX == 0, "unroll must align ring and X buffers");
    static_assert(kWaves * NT * 256 <= 256 * 64, "partial tiles must fit the table's LDS");

    // 64 KiB: the lane-replicated code table, then the partial tiles
    __shared__ uint32_t s_lds[256 * 64];
    __shared__ float s_lv[16];
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
    if constexpr (kDQ) {
        st.q = rsrc(w.q + n_base * nblk, rows * nblk);
        // the groups holding the workgroup's blocks
        const int64_t g0 = n_base * nblk / 256, g1 = ((n_base + rows) * nblk - 1) / 256;
        st.sc = rsrc(w.scale + g0, (g1 - g0 + 1) * 4);
        st.q_off = (uint32_t)(r * nblk);
    } else {
        st.q = rsrc(w.absmax + n_base * nblk, rows * nblk * 4);
        st.q_off = (uint32_t)(r * nblk * 4);
    }
    st.x = rsrc(x, (int64_t)m * K * 2);
    st.c_off = (uint32_t)(r * (K / 2) + 16 * g);
    st.flat0 = (uint32_t)((n_base + r) * nblk - (n_base * nblk / 256) * 256);
    st.x_off = (uint32_t)(2 * (r * K + 16 * sg));

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
            if (u0 + J < units)
                unit_mac<kDQ, kMI>(acc[t], ring[J % kRing], xa[ci % kNX], xb[ci % kNX], lds, lane4);
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

}  // namespace

// The descriptors address each workgroup's rows with 32-bit offsets:
// 128 rows of K/2 bytes, and 16 rows of X.
bool gemv_supported(int64_t m, int64_t k) {
    return m >= 1 && m <= 16 && k % kChunk == 0 && k <= (int64_t)1 << 24;
}

hipError_t launch_gemv(const uint16_t *x, int64_t m, const nf4_weight &wt, uint16_t *y, hipStream_t s) {
    const WView w = make_view(wt);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t tiles = (w.n + 15) / 16;
    const int nt = (int)std::min<int64_t>(std::max<int64_t>((tiles + cus - 1) / cus, 1), kMaxNT);
    const dim3 grid((unsigned)((tiles + nt - 1) / nt));
    if (m == 1)
        launch_mi<1>(nt, grid, x, (int)m, w, y, s);
    else
        launch_mi<4>(nt, grid, x, (int)m, w, y, s);
    return hipGetLastError();
}

}  // namespace nf4
