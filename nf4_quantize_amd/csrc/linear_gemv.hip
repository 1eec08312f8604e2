// linear_gemv.hip - decode-shaped fused NF4 linear (M <= 16 activation rows)
// for gfx950: Y[M x N] = X[M x K] . dequantize(W)^T, W stored [N x K] NF4
// ([MF] "Forward Pass Computation"; source key in nf4_internal.h).
//
// The weight is streamed once from HBM and never materialised. X is padded
// to 16 rows and the contraction runs on v_mfma_f32_16x16x32_bf16 with
// A = X rows and B = 16 weight rows (16 output columns). Lane l = 16 g + r
// holds row r of both operands; within a 64-block it owns the 16 contiguous
// weights k = 64 b + 16 g + [0, 16), split over the block's two MFMA steps.
// The pairing of k across lanes is the same for A and B, so the products are
// exactly those of the dot product, and both steps stay inside one block:
// the block's MFMA sum is scaled afterwards by its c1' (4 FMAs per lane per
// block instead of a multiply per weight).
//
// Codes become bf16 pairs through a 256-entry table (byte -> (q[lo], q[hi])
// rounded to bf16) held in LDS once per lane: entry e of lane l is the word
// at byte 256 e + 4 l, so a lane always reads its own bank and the
// data-dependent lookups never conflict. One v_perm_b32 builds each address
// (byte k of the code word next to the lane offset).
//
// Work split: a workgroup of kWaves waves owns NT tiles of 16 output columns
// and all of K. Wave w owns 1/kWaves of each K super-chunk: its slice of X is
// loaded into registers once and reused for the NT tiles, whose codes stream
// through a kRing-deep register ring; each wave keeps its NT partial tiles in
// registers and the partials are summed once, through LDS, at the end. NT is
// chosen so that the grid is about one workgroup per CU.
#include <algorithm>

#include "linear_common.h"

namespace nf4 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBpw = 4;     // blocks per wave per super-chunk
constexpr int kMaxNT = 8;   // column tiles per workgroup
// Waves per workgroup (the K split) and depth of the per-wave ring of tile
// loads. 8 waves leave a 256-register budget per wave, so NT tiles of
// accumulators and a deep ring fit without spills.
constexpr int kWaves = 8;
constexpr int kRing = 3;
constexpr int kWgPerCu = 1;  // target resident workgroups per CU when sizing NT
constexpr bool kPrefetchX = false;  // fetch X of the next super-chunk ahead (double buffer)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// One tile's operands for this lane: the codes of kBpw blocks of weight row
// n and their raw scale data (decoded at use, so that issuing the loads never
// waits on earlier ones): E4M3 codes and the group's c2 with double
// quantization, else the fp32 absmax values.
template <bool kDQ> struct TileCodes;
template <> struct TileCodes<true> {
    u32x2_t c[kBpw];
    uint32_t q8;
    float c2;
};
template <> struct TileCodes<false> {
    u32x2_t c[kBpw];
    f32x4 am;
};

// Per-lane base addresses of this wave's blocks in the workgroup's first
// tile; tile t is 16 weight rows further (a uniform stride).
struct TileBase {
    const uint8_t *codes;   // row n_base + r, byte of block b0, lane group g
    uint64_t flat;          // flat block index (n_base + r) * nblk + b0
    int64_t n;              // weight row n_base + r
};

// Requires K % 256 == 0: the 4 blocks of a tile then share one 4-byte-aligned
// word of scale codes and one group.
template <bool kDQ>
__device__ __forceinline__ void load_tile(TileCodes<kDQ> &tc, const WView &w, const TileBase &tb, int t) {
    const uint64_t nblk = (uint64_t)w.k / kBlock;
#pragma unroll
    for (int j = 0; j < kBpw; ++j) tc.c[j] = u32x2_t{0x77777777u, 0x77777777u};  // code 7 = 0.0
    if constexpr (kDQ) {
        tc.q8 = 0;
        tc.c2 = 0.0f;
    } else {
        tc.am = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (tb.n + 16 * t < w.n) {
        const uint8_t *rowc = tb.codes + (uint64_t)(16 * t) * ((uint64_t)w.k / 2);
#pragma unroll
        for (int j = 0; j < kBpw; ++j) tc.c[j] = *reinterpret_cast<const u32x2_t *>(rowc + 32 * j);
        const uint64_t flat = tb.flat + (uint64_t)(16 * t) * nblk;
        if constexpr (kDQ) {
            tc.q8 = *reinterpret_cast<const uint32_t *>(w.q + flat);
            tc.c2 = w.scale[flat >> 8];
        } else {
            tc.am = *reinterpret_cast<const f32x4 *>(w.absmax + flat);
        }
    }
}

__device__ __forceinline__ TileBase tile_base(const WView &w, int64_t n_base, int r, int g, int64_t b0) {
    const int64_t n = n_base + r;
    TileBase tb;
    tb.codes = w.codes + (uint64_t)n * ((uint64_t)w.k / 2) + (uint64_t)b0 * 32 + 8 * g;
    tb.flat = (uint64_t)n * ((uint64_t)w.k / kBlock) + (uint64_t)b0;
    tb.n = n;
    return tb;
}

template <bool kDQ, int J>
__device__ __forceinline__ float tile_scale(const TileCodes<kDQ> &tc) {
    // gfx950's fp8 -> f32 convert decodes OCP E4M3FN exactly
    if constexpr (kDQ) return __builtin_amdgcn_cvt_f32_fp8((int)tc.q8, J) * tc.c2;
    else return tc.am[J];
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

// One tile (4 blocks of 16 weight rows) in two halves: each half issues the
// table lookups of 2 blocks, then their 4 MFMAs (2 independent chains), then
// the per-block scaling.
template <bool kDQ, int H>
__device__ __forceinline__ void half_mac(f32x4_t &acc, const TileCodes<kDQ> &tc, const u32x4 (&xa)[kBpw],
                                         const u32x4 (&xb)[kBpw], const char *lds, uint32_t lane4) {
    constexpr int J0 = 2 * H, J1 = 2 * H + 1;
    const u32x4 lo0 = lookup4(lds, tc.c[J0].x, lane4), hi0 = lookup4(lds, tc.c[J0].y, lane4);
    const u32x4 lo1 = lookup4(lds, tc.c[J1].x, lane4), hi1 = lookup4(lds, tc.c[J1].y, lane4);
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[J0]), as_bf16x8(lo0), z, 0, 0, 0);
    f32x4_t p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[J1]), as_bf16x8(lo1), z, 0, 0, 0);
    p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb[J0]), as_bf16x8(hi0), p0, 0, 0, 0);
    p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xb[J1]), as_bf16x8(hi1), p1, 0, 0, 0);
    // D row 4 g + i, column r: that column is weight row n, scaled by c1'(n, b)
    acc += p0 * tile_scale<kDQ, J0>(tc);
    acc += p1 * tile_scale<kDQ, J1>(tc);
}

template <bool kDQ>
__device__ __forceinline__ void tile_mac(f32x4_t &acc, const TileCodes<kDQ> &tc, const u32x4 (&xa)[kBpw],
                                         const u32x4 (&xb)[kBpw], const char *lds, uint32_t lane4) {
    half_mac<kDQ, 0>(acc, tc, xa, xb, lds, lane4);
    half_mac<kDQ, 1>(acc, tc, xa, xb, lds, lane4);
}

__device__ __forceinline__ void load_x(u32x4 (&xa)[kBpw], u32x4 (&xb)[kBpw], const uint16_t *x,
                                       bool has_x, int r, int g, int64_t K, int64_t b0) {
#pragma unroll
    for (int j = 0; j < kBpw; ++j) {
        xa[j] = u32x4{0, 0, 0, 0};
        xb[j] = u32x4{0, 0, 0, 0};
        if (has_x) {
            const u32x4 *xp = reinterpret_cast<const u32x4 *>(x + (int64_t)r * K + (b0 + j) * kBlock + 16 * g);
            xa[j] = xp[0];
            xb[j] = xp[1];
        }
    }
}

template <int NT, bool kDQ>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(const uint16_t *__restrict__ x, int m,
                                                           WView w, uint16_t *__restrict__ y,
                                                           Levels lv) {
    // 64 KiB: the lane-replicated code table, then the partial tiles
    static_assert(64 % kWaves == 0, "reduction rounds assume kWaves divides 64");
    __shared__ uint32_t s_lds[256 * 64];
    const char *lds = reinterpret_cast<const char *>(s_lds);

    const int tid = threadIdx.x;
    for (int i = tid; i < 256 * 64; i += 64 * kWaves) {
        const int e = i >> 6;
        s_lds[i] = pack_bf16x2(lv.q[e & 15], lv.q[e >> 4]);
    }
    __syncthreads();

    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const uint32_t lane4 = 4u * lane;
    const int64_t K = w.k, nblk = K / kBlock;
    const int64_t n_base = (int64_t)blockIdx.x * 16 * NT;
    const bool has_x = r < m;

    f32x4_t acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // This wave's K blocks: b0 = wave * kBpw + s * kWaves * kBpw for super-chunk
    // s (all 4 blocks exist because K % 256 == 0). Tiles stream through a
    // ring that runs across super-chunk boundaries; X of the next super-chunk
    // is fetched while the current one computes.
    const int64_t step = (int64_t)kWaves * kBpw;
    int64_t b0 = (int64_t)wave * kBpw;
    if (b0 < nblk) {
        u32x4 xa[kBpw], xb[kBpw], xna[kBpw], xnb[kBpw];
        load_x(xa, xb, x, has_x, r, g, K, b0);
        TileCodes<kDQ> ring[kRing];
        TileBase tb = tile_base(w, n_base, r, g, b0);
#pragma unroll
        for (int t = 0; t < kRing - 1; ++t)
            if (t < NT) load_tile<kDQ>(ring[t], w, tb, t);
        for (;;) {
            const int64_t b_next = b0 + step;
            const bool more = b_next < nblk;
            if (kPrefetchX && more) load_x(xna, xnb, x, has_x, r, g, K, b_next);
            const TileBase tbn = tile_base(w, n_base, r, g, more ? b_next : b0);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                // keep kRing - 1 tiles in flight, continuing into the next super-chunk
                const int ahead = t + kRing - 1;
                if (ahead < NT)
                    load_tile<kDQ>(ring[ahead % kRing], w, tb, ahead);
                else if (more && ahead - NT < NT)
                    load_tile<kDQ>(ring[ahead % kRing], w, tbn, ahead - NT);
                tile_mac<kDQ>(acc[t], ring[t % kRing], xa, xb, lds, lane4);
            }
            if (!more) break;
            // the ring slots consumed next start at index NT % kRing: rotate so
            // that the next super-chunk's tile t sits in ring[t % kRing]
            if (NT % kRing != 0) {
                TileCodes<kDQ> tmp[kRing];
#pragma unroll
                for (int i = 0; i < kRing; ++i) tmp[i] = ring[(i + NT) % kRing];
#pragma unroll
                for (int i = 0; i < kRing; ++i) ring[i] = tmp[i];
            }
            if (kPrefetchX) {
#pragma unroll
                for (int j = 0; j < kBpw; ++j) {
                    xa[j] = xna[j];
                    xb[j] = xnb[j];
                }
            } else {
                load_x(xa, xb, x, has_x, r, g, K, b_next);
            }
            b0 = b_next;
            tb = tbn;
        }
    }

    // Sum the waves' partial tiles through LDS, TPR tiles per round: the
    // 16384-word table holds kWaves x TPR tiles of 256 floats.
    constexpr int TPR = 64 / kWaves;
    float *red = reinterpret_cast<float *>(s_lds);  // [wave][TPR tiles][4][64]
#pragma unroll
    for (int t0 = 0; t0 < NT; t0 += TPR) {
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < TPR; ++tt)
            if (t0 + tt < NT)
#pragma unroll
                for (int i = 0; i < 4; ++i) red[((wave * TPR + tt) * 4 + i) * 64 + lane] = acc[t0 + tt][i];
        __syncthreads();
        for (int e = tid; e < TPR * 256; e += 64 * kWaves) {
            const int tt = e >> 8, i = (e >> 6) & 3, l = e & 63;
            if (t0 + tt < NT) {
                float s = 0.0f;
#pragma unroll
                for (int v = 0; v < kWaves; ++v) s += red[((v * TPR + tt) * 4 + i) * 64 + l];
                const int64_t n = n_base + 16 * (t0 + tt) + (l & 15);
                const int row = 4 * (l >> 4) + i;
                if (row < m && n < w.n) y[(int64_t)row * w.n + n] = (uint16_t)(pack_bf16x2(s, 0.0f) & 0xFFFFu);
            }
        }
    }
}

template <int NT>
void launch_nt(dim3 grid, const uint16_t *x, int m, const WView &w, uint16_t *y, hipStream_t s) {
    if (w.q)
        gemv_kernel<NT, true><<<grid, dim3(64 * kWaves), 0, s>>>(x, m, w, y, levels());
    else
        gemv_kernel<NT, false><<<grid, dim3(64 * kWaves), 0, s>>>(x, m, w, y, levels());
}

}  // namespace

bool gemv_supported(int64_t m, int64_t k) { return m >= 1 && m <= 16 && k % 256 == 0; }

hipError_t launch_gemv(const uint16_t *x, int64_t m, const nf4_weight &wt, uint16_t *y,
                       hipStream_t s) {
    const WView w = make_view(wt);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t tiles = (w.n + 15) / 16;
    const int64_t slots = (int64_t)cus * kWgPerCu;
    const int nt = (int)std::min<int64_t>(std::max<int64_t>((tiles + slots - 1) / slots, 1), kMaxNT);
    const dim3 grid((unsigned)((tiles + nt - 1) / nt));
    switch (nt) {
        case 1: launch_nt<1>(grid, x, (int)m, w, y, s); break;
        case 2: launch_nt<2>(grid, x, (int)m, w, y, s); break;
        case 3: launch_nt<3>(grid, x, (int)m, w, y, s); break;
        case 4: launch_nt<4>(grid, x, (int)m, w, y, s); break;
        case 5: launch_nt<5>(grid, x, (int)m, w, y, s); break;
        case 6: launch_nt<6>(grid, x, (int)m, w, y, s); break;
        case 7: launch_nt<7>(grid, x, (int)m, w, y, s); break;
        default: launch_nt<8>(grid, x, (int)m, w, y, s); break;
    }
    return hipGetLastError();
}

}  // namespace nf4
