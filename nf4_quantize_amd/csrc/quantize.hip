// quantize.hip - blockwise NF4 quantization with fused double quantization
// for gfx950 ([MF] "Block-Wise Quantization Mechanics" and "Double
// Quantization (DQ)", see nf4_internal.h for the source key).
//
// Work split: one workgroup of 512 threads per group of 256 blocks (16384
// weights), so c2 = max c1 of the group is a workgroup reduction and never
// leaves the chip. Each lane owns one 16-byte slice of a block (8 bf16 or 4
// fp32 weights); consecutive lanes own consecutive slices, so every wave
// load is one contiguous 1 KiB run. A block's absmax is a DPP max across the
// 8 (bf16) or 16 (fp32) lanes that hold it.
//
// The nearest level is found without a 16-way search: n = fl(w / c1) is
// approximated by x = w * rcp(c1), which is bucketed (one fma + mask) into a
// 33-entry LDS table giving the bucket's switch point thr and top code hi;
// the code is hi - (x < thr), with d = x - thr from one more fma. x differs
// from n by < 1.5e-7; lanes with |d| < 2^-20 redo their slice with the
// correctly rounded division, so codes are exactly those of the definition.
// The table is held in 8 (bf16) or 4 (fp32) copies, copy e with hi shifted to
// nibble e, so a slice's codes are the OR of its entries' hi fields minus the
// sign bits of its d values gathered to nibble positions.
#pragma clang fp contract(off)

#include <algorithm>
#include <type_traits>

#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

// Max of non-negative floats via their bit patterns (monotone as unsigned),
// with the neighbour lane brought in by DPP (0 is the identity of the max, so
// the move folds into the max instruction).
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, 0xF, 0xF, true));
}

// Max over the wave of non-negative floats, returned to every lane: DPP
// within each row of 16 lanes, then the four row results by v_readlane.
__device__ __forceinline__ float wave_max_nonneg(float x) {
    uint32_t v = __float_as_uint(x);
    v = dpp_umax<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_umax<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_umax<0x141>(v);  // row_half_mirror
    v = dpp_umax<0x140>(v);  // row_mirror
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return __uint_as_float(max(a, b));
}

// Max over the whole workgroup of T threads of non-negative floats; every
// thread gets the result.
template <int T = kThreads>
__device__ __forceinline__ float wg_max(float v, float *s_red) {
    const float m = wave_max_nonneg(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_red[wave] = m;
    __syncthreads();
    float r = s_red[0];
#pragma unroll
    for (int i = 1; i < T / 64; ++i) r = fmaxf(r, s_red[i]);
    return r;
}

// Pairwise fp32 sum of s_v[0..255], the subtree of a pairwise sum that an
// aligned run of 256 values forms: threads 0..255 hold one value each, lanes
// pair up by XOR shuffles (x + y == y + x, so both lanes of a pair hold the
// node), and the four wave sums pair last. Every thread of the workgroup
// calls it; the result is valid in all of them.
__device__ __forceinline__ float block256_pairwise_sum(const float *s_v, float *s_red) {
    const int t = threadIdx.x;
    float v = t < 256 ? s_v[t] : 0.0f;
#pragma unroll
    for (int k = 1; k < 64; k *= 2) v = v + __shfl_xor(v, k);
    if ((t & 63) == 0 && t < 256) s_red[t >> 6] = v;
    __syncthreads();
    return (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
}

// Byte offset of the table entry of a normalised value (see CodeLut).
__device__ __forceinline__ uint32_t lut_offset(float v) {
    return lut_offset_bits(fmaf(v, 128.0f, 128.0f + 0x1p23f));
}
__device__ __forceinline__ float2 lut_at(const float2 *s_lut, uint32_t off) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(s_lut) + off);
}
// Code of an exactly normalised value (the definition's fl32(w / c1)); with
// a sign-magnitude table (CodeLut::signmag), the code of |nrm| plus 8 for a
// negative value with a non-zero magnitude code.
__device__ __forceinline__ uint32_t exact_code(const float2 *s_lut, float nrm, bool signmag = false) {
    const float v = signmag ? fabsf(nrm) : nrm;
    const float2 ent = lut_at(s_lut, lut_offset(v));
    const uint32_t c = (uint32_t)__float_as_int(ent.y) - (v < ent.x ? 1u : 0u);
    return (signmag && c != 0u && signbit(nrm)) ? c + 8u : c;
}

// Input traits: one 16-byte slice per lane.
template <typename T> struct Slice;
template <> struct Slice<uint16_t> {  // bf16
    static constexpr int kElems = 8;
    using Vec = u32x4;
    __device__ static void widen(const Vec &v, float (&f)[8]) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
};
template <> struct Slice<float> {
    static constexpr int kElems = 4;
    using Vec = f32x4;
    __device__ static void widen(const Vec &v, float (&f)[4]) {
        f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
    }
};

// Bit 4e of the result is the sign bit of d[e] (E = 4 or 8). v_perm_b32
// selectors 9 and 11 give a byte of copies of bit 31 of the second and the
// first source, 12 a zero byte: each v_perm gathers two signs.
template <int E>
__device__ __forceinline__ uint32_t sign_nibbles(const float (&d)[E]) {
    auto u = [&](int e) { return __float_as_uint(d[e]); };
    if constexpr (E == 8) {
        const uint32_t ev = __builtin_amdgcn_perm(u(2), u(0), 0x0C0C0B09u) |
                            __builtin_amdgcn_perm(u(6), u(4), 0x0B090C0Cu);
        const uint32_t od = __builtin_amdgcn_perm(u(3), u(1), 0x0C0C0B09u) |
                            __builtin_amdgcn_perm(u(7), u(5), 0x0B090C0Cu);
        return (ev & 0x01010101u) | (od & 0x10101010u);
    } else {
        const uint32_t ev = __builtin_amdgcn_perm(u(2), u(0), 0x0C0C0B09u);
        const uint32_t od = __builtin_amdgcn_perm(u(3), u(1), 0x0C0C0B09u);
        return (ev & 0x0101u) | (od & 0x1010u);
    }
}

// Packed sign-magnitude codes: packed holds the magnitude codes (each below
// 8), and the code of a negative weight with a non-zero magnitude code gets
// bit 3 of its nibble (see CodeLut::signmag). Adding 7 to a nibble below 8
// sets its bit 3 exactly when it is non-zero, with no carry between nibbles.
template <int E>
__device__ __forceinline__ uint32_t apply_signs(uint32_t packed, const float (&f)[E]) {
    const uint32_t nonzero = (packed + 0x77777777u) & 0x88888888u;
    return packed | (nonzero & (sign_nibbles<E>(f) << 3));
}

// Codes of one lane's slice. c1 is the block absmax (all lanes of the block
// hold the same value). s_lut holds E copies of the table, copy e with the
// top code shifted to nibble e. Returns the packed nibbles, element e at
// bits 4e. SM: a sign-magnitude table, looked up with |w|.
template <int E, bool SM = false>
__device__ __forceinline__ uint32_t slice_codes(const float (&f)[E], float c1, const float2 *s_lut) {
    // rcp ~ 1/c1 from v_rcp_f32 (within 1 ulp for a normal result). With
    // x = w * rcp as a real number, |x - fl(w/c1)| < 1.5e-7 for |w| <= c1.
    // The bucket is that of x (one fma with 128 rcp, a power-of-two multiple)
    // and d = fl(x - thr) (one fma). Whenever |d| >= kNearTol, x and
    // fl(w/c1) lie on the same side of thr, and as every switch point sits
    // at least 2^-16 inside its bucket, x's entry gives fl(w/c1)'s code.
    // Blocks with c1 == 0 (all zero) take rcp = 0 (x = 0 -> code 7). A c1
    // outside [2^-118, 2^125] - where 128 rcp would overflow, or rcp fall
    // into the subnormal range where v_rcp_f32 is not that accurate - takes
    // the exact path for the whole slice.
    const bool in_range = (c1 >= 0x1p-118f) & (c1 <= 0x1p125f);
    const bool outside = (c1 > 0.0f) & !in_range;
    const float rcp = in_range ? __builtin_amdgcn_rcpf(c1) : 0.0f;
    const float rcp128 = rcp * 128.0f;
    uint32_t top = 0;
    float d[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float fe = SM ? fabsf(f[e]) : f[e];
        const float2 ent = lut_at(s_lut + e * kLutEntries,
                                  lut_offset_bits(fmaf(fe, rcp128, 128.0f + 0x1p23f)));
        d[e] = fmaf(fe, rcp, -ent.x);
        top |= __float_as_uint(ent.y);
    }
    float dmin = fabsf(d[0]);
#pragma unroll
    for (int e = 1; e < E; ++e) dmin = fminf(dmin, fabsf(d[e]));
    uint32_t packed = top - sign_nibbles<E>(d);
    if (SM) packed = apply_signs<E>(packed, f);
    if (outside | !(dmin >= kNearTol)) {  // rare: redo with the correctly rounded division
        packed = 0;
#pragma unroll
        for (int e = 0; e < E; ++e)
            packed |= exact_code(s_lut, c1 > 0.0f ? f[e] / c1 : 0.0f, SM) << (4 * e);
    }
    return packed;
}

// Codes of a bf16 slice for the codebooks with `refine` set (see CodeLut).
// One residual step makes the quotient exact: with rcp within 1 ulp of 1/c1,
// x = fl(w rcp) and r = fma(-c1, x, w), the value x + r rcp is within
// 2^-22 ulp of w / c1, while the quotient of two bf16 values (8-bit
// significands) is never a rounding midpoint and lies at least 2^-9 ulp from
// one. So xr = fma(r, rcp, x) = fl32(w / c1), and the switch point test
// xr < thr is exact. Quotients below 2^-120 (subnormal results round on a
// coarser grid) and a c1 outside [2^-118, 2^125] take the division.
template <bool SM>
__device__ __forceinline__ uint32_t slice_codes_refined(const float (&f)[8], float c1,
                                                        const float2 *s_lut) {
    const bool in_range = (c1 >= 0x1p-118f) & (c1 <= 0x1p125f);
    const bool outside = (c1 > 0.0f) & !in_range;
    const float rcp = in_range ? __builtin_amdgcn_rcpf(c1) : 0.0f;
    uint32_t top = 0;
    bool tiny = false;
    float d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = f[e] * rcp;
        const float r = fmaf(-c1, x, f[e]);
        const float xr = fmaf(r, rcp, x);
        const float xe = SM ? fabsf(xr) : xr;
        const float2 ent = lut_at(s_lut + e * kLutEntries,
                                  lut_offset_bits(fmaf(xe, 128.0f, 128.0f + 0x1p23f)));
        d[e] = xe - ent.x;  // negative exactly when xe < thr
        top |= __float_as_uint(ent.y);
        tiny |= ((__float_as_uint(xr) & 0x7FFFFFFFu) - 1u) < 0x037FFFFFu;  // 0 < |xr| < 2^-120
    }
    uint32_t packed = top - sign_nibbles<8>(d);
    if (SM) packed = apply_signs<8>(packed, f);
    if (outside | tiny) {  // rare: redo with the correctly rounded division
        packed = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            packed |= exact_code(s_lut, c1 > 0.0f ? f[e] / c1 : 0.0f, SM) << (4 * e);
    }
    return packed;
}

// Codes of a slice, refined for the codebooks that need it (bf16 only; an
// fp32 quotient can sit next to a midpoint, so fp32 slices keep the
// division fallback).
template <int E>
__device__ __forceinline__ uint32_t slice_codes_any(const float (&f)[E], float c1,
                                                    const float2 *s_lut, const CodeLut &lut) {
    if constexpr (E == 8) {
        if (lut.refine)
            return lut.signmag ? slice_codes_refined<true>(f, c1, s_lut)
                               : slice_codes_refined<false>(f, c1, s_lut);
    }
    return lut.signmag ? slice_codes<E, true>(f, c1, s_lut) : slice_codes<E, false>(f, c1, s_lut);
}

// Codebook kinds, fixed at compile time in the group kernels so that each
// kernel holds one slice path: bit 0 a sign-magnitude table (CodeLut::signmag),
// bit 1 the refined bf16 quotient (CodeLut::refine; fp32 slices keep the
// division fallback, so the bit is dropped for them).
template <typename T>
int cb_kind(const CodeLut &lut) {
    return (lut.signmag ? 1 : 0) | ((sizeof(T) == 2 && lut.refine) ? 2 : 0);
}

// slice_codes_any with the codebook kind CB fixed.
template <int E, int CB>
__device__ __forceinline__ uint32_t slice_codes_cb(const float (&f)[E], float c1, const float2 *s_lut) {
    constexpr bool SM = (CB & 1) != 0;
    if constexpr (E == 8 && (CB & 2) != 0)
        return slice_codes_refined<SM>(f, c1, s_lut);
    else
        return slice_codes<E, SM>(f, c1, s_lut);
}

// Calls fn(std::integral_constant<int, CB>()) for the codebook kind of lut.
template <typename T, typename Fn>
hipError_t with_cb(const CodeLut &lut, Fn &&fn) {
    const int k = cb_kind<T>(lut);
    if (k == 1) return fn(std::integral_constant<int, 1>());
    if constexpr (sizeof(T) == 2) {
        if (k == 2) return fn(std::integral_constant<int, 2>());
        if (k == 3) return fn(std::integral_constant<int, 3>());
    }
    return fn(std::integral_constant<int, 0>());
}

// Entry i of the table copies (copy i / kLutEntries, see slice_codes).
__device__ __forceinline__ float2 lut_copy_entry(const LutEntry &le, int i) {
    return make_float2(le.thr, __int_as_float(le.hi << (4 * (i / kLutEntries))));
}

__device__ __forceinline__ void load_lut(const CodeLut &lut, float2 *s_lut) {
    if (threadIdx.x < kLutEntries) s_lut[threadIdx.x] = lut_copy_entry(lut.e[threadIdx.x], 0);
}

// The stored group value of unsigned codes: c2, or the linear code's step.
template <int F>
__device__ __forceinline__ float group_value(float c2) {
    return F == kFmtLin8 ? c2 / lin_levels<false>() : c2;
}

// Double quantization of a group's 256 block scales: s_c1 holds them and
// s_red the maxima of the workgroup's waves (so c2 is their max); threads
// 0..63 each encode 4 consecutive blocks as one 32-bit store of 8-bit codes
// in format F.
template <int T, int F>
__device__ __forceinline__ void group_dq(const float *s_c1, const float *s_red, uint8_t *absmax_q,
                                         float *absmax_scale, int64_t g) {
    const int t = threadIdx.x;
    if (t >= kDqBlock / 4) return;
    float c2 = s_red[0];
#pragma unroll
    for (int i = 1; i < T / 64; ++i) c2 = fmaxf(c2, s_red[i]);
    const float sc = group_value<F>(c2);
    const float4 c = reinterpret_cast<const float4 *>(s_c1)[t];
    const uint32_t q = dq_encode<F, false>(c.x, sc) | (dq_encode<F, false>(c.y, sc) << 8) |
                       (dq_encode<F, false>(c.z, sc) << 16) | (dq_encode<F, false>(c.w, sc) << 24);
    reinterpret_cast<uint32_t *>(absmax_q + g * kDqBlock)[t] = q;
    if (t == 0) absmax_scale[g] = sc;
}

// LDS of one group in flight: its codes, gathered for 16-byte stores, its
// 256 block scales and the maxima of the workgroup's waves.
template <int TH>
struct GroupLds {
    u32x4 codes[kGroup / 32];
    float c1[kDqBlock];
    float red[TH / 64];
};

// The table copies of slice_codes in LDS, from the argument block: entry
// t % kTab for thread t (threads past the table store a duplicate).
template <int E, int TH>
__device__ __forceinline__ void store_lut(const LutEntry &le, float2 *s_lut) {
    constexpr int kTab = E * kLutEntries;
    static_assert(kTab <= TH, "one table entry per thread");
    s_lut[threadIdx.x % kTab] = lut_copy_entry(le, threadIdx.x % kTab);
}

// Codes and block scales of group g, whose weights thread t holds in v
// (slices t, t + TH, ...). Writes the codes and the block scales to L, the
// wave maxima too with double quantization, and the block scales to absmax
// if set. The caller's barrier then publishes L to group_finish.
template <typename T, bool kDQ, int TH, int CB>
__device__ __forceinline__ void group_codes(const typename Slice<T>::Vec (&v)[kGroup / Slice<T>::kElems / TH],
                                            GroupLds<TH> &L, float *__restrict__ absmax,
                                            const float2 *s_lut, bool keep_c1, const int64_t g) {
    using S = Slice<T>;
    constexpr int E = S::kElems;               // weights per lane slice
    constexpr int LPB = kBlock / E;            // lanes per block
    constexpr int ITERS = kGroup / E / TH;     // slices per thread
    constexpr int BPI = TH / LPB;              // blocks per iteration
    const int t = threadIdx.x;
    float mmax = 0.0f;  // max of this thread's block scales
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        float f[E];
        S::widen(v[i], f);
        float mf = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) mf = fmaxf(mf, fabsf(f[e]));
        uint32_t mb = __float_as_uint(mf);
        mb = dpp_umax<0xB1>(mb);   // quad_perm [1,0,3,2]
        mb = dpp_umax<0x4E>(mb);   // quad_perm [2,3,0,1]
        mb = dpp_umax<0x141>(mb);  // row_half_mirror: lanes i <-> 7-i
        if (LPB == 16) mb = dpp_umax<0x140>(mb);  // row_mirror: lanes i <-> 15-i
        const float m = __uint_as_float(mb);
        mmax = fmaxf(mmax, m);
        const int blk = i * BPI + t / LPB;  // block within the group
        if ((t % LPB) == 0) {
            if (kDQ || keep_c1) L.c1[blk] = m;
            if (absmax) absmax[g * kDqBlock + blk] = m;
        }
        const uint32_t packed = slice_codes_cb<E, CB>(f, m, s_lut);
        if (E == 8)
            reinterpret_cast<uint32_t *>(L.codes)[i * TH + t] = packed;
        else
            reinterpret_cast<uint16_t *>(L.codes)[i * TH + t] = (uint16_t)packed;
    }
    if (kDQ) {
        const float wm = wave_max_nonneg(mmax);
        if ((t & 63) == 0) L.red[t >> 6] = wm;
    }
}

// After the barrier that follows group_codes: the group's codes, 16 bytes
// per thread (each wave one contiguous 1 KiB run), and its double
// quantization.
template <bool kDQ, int TH, int F>
__device__ __forceinline__ void group_finish(const GroupLds<TH> &L, uint8_t *__restrict__ codes,
                                             uint8_t *__restrict__ absmax_q,
                                             float *__restrict__ absmax_scale, const int64_t g) {
    static_assert(kGroup / 32 == TH, "one 16-byte piece of the group's codes per thread");
    __builtin_nontemporal_store(L.codes[threadIdx.x],
                                reinterpret_cast<u32x4 *>(codes + g * (kGroup / 2)) + threadIdx.x);
    if (kDQ) group_dq<TH, F>(L.c1, L.red, absmax_q, absmax_scale, g);
}

// Full group g of a tensor, by a workgroup of TH threads. Without fused
// double quantization, `partial` (if set) receives the pairwise sum of the
// group's 256 block scales (the first levels of the mean offset's sum).
template <typename T, bool kDQ, int TH, int F, int CB>
__device__ __forceinline__ void quantize_group(
    const T *__restrict__ w, uint8_t *__restrict__ codes, float *__restrict__ absmax,
    uint8_t *__restrict__ absmax_q, float *__restrict__ absmax_scale, float *__restrict__ partial,
    const CodeLut &lut, const int64_t g) {
    using S = Slice<T>;
    constexpr int ITERS = kGroup / S::kElems / TH;
    __shared__ float2 s_lut[S::kElems * kLutEntries];
    __shared__ __align__(16) GroupLds<TH> L;

    const int t = threadIdx.x;
    const typename S::Vec *src = reinterpret_cast<const typename S::Vec *>(w + g * kGroup);
    // The table comes from the argument block through a vector load: issued
    // first and stored to LDS after the weight loads are on their way, so its
    // wait does not cover them.
    const LutEntry le = lut.e[t % kLutEntries];
    __builtin_amdgcn_sched_barrier(0);
    typename S::Vec v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) v[i] = __builtin_nontemporal_load(&src[i * TH + t]);
    store_lut<S::kElems, TH>(le, s_lut);
    __syncthreads();
    group_codes<T, kDQ, TH, CB>(v, L, absmax, s_lut, partial != nullptr, g);
    __syncthreads();
    group_finish<kDQ, TH, F>(L, codes, absmax_q, absmax_scale, g);
    if (!kDQ && partial) {
        const float sum = block256_pairwise_sum(L.c1, L.red);
        if (t == 0) partial[g] = sum;
    }
}

// One workgroup per full group of 16384 weights.
template <typename T, bool kDQ, int TH, int F, int CB>
__global__ __launch_bounds__(TH) void quantize_groups_kernel(
    const T *__restrict__ w, uint8_t *__restrict__ codes, float *__restrict__ absmax,
    uint8_t *__restrict__ absmax_q, float *__restrict__ absmax_scale, float *__restrict__ partial,
    CodeLut lut) {
    quantize_group<T, kDQ, TH, F, CB>(w, codes, absmax, absmax_q, absmax_scale, partial, lut,
                                  (int64_t)blockIdx.x);
}

// The final partial group g of an n-element tensor: thread t owns block t of
// the group and works element by element with guarded accesses.
template <typename T, int F>
__device__ __forceinline__ void quantize_tail(
    const T *__restrict__ w, int64_t n, int64_t g, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, uint8_t *__restrict__ absmax_q, float *__restrict__ absmax_scale,
    float *__restrict__ partial, const CodeLut &lut) {
    __shared__ float2 s_lut[kLutEntries];
    __shared__ float s_c1[kDqBlock];
    __shared__ float s_red[4];
    const int t = threadIdx.x;
    load_lut(lut, s_lut);
    __syncthreads();
    const int64_t b = g * kDqBlock + t;
    const int64_t lo = b * kBlock;
    const int64_t hi = min(lo + kBlock, n);
    auto elem = [&](int64_t i) -> float {
        if constexpr (sizeof(T) == 2) return __uint_as_float((uint32_t)w[i] << 16);
        else return w[i];
    };
    float c1 = 0.0f;
    for (int64_t i = lo; i < hi; ++i) c1 = fmaxf(c1, fabsf(elem(i)));
    s_c1[t] = c1;
    if (lo < n && absmax) absmax[b] = c1;
    for (int64_t i = lo; i < hi; i += 2) {
        uint32_t byte = 0;
        for (int j = 0; j < 2 && i + j < hi; ++j) {
            const uint32_t code = exact_code(s_lut, (c1 > 0.0f) ? elem(i + j) / c1 : 0.0f, lut.signmag != 0);
            byte |= code << (4 * j);
        }
        codes[i / 2] = (uint8_t)byte;
    }
    if (absmax_q) {
        __syncthreads();
        const float sc = group_value<F>(wg_max(s_c1[t], s_red));
        const int64_t nblocks = (n + kBlock - 1) / kBlock;
        if (b < nblocks) absmax_q[b] = (uint8_t)dq_encode<F, false>(s_c1[t], sc);
        if (t == 0) absmax_scale[g] = sc;
    } else if (partial) {
        __syncthreads();
        const float sum = block256_pairwise_sum(s_c1, s_red);  // blocks past n hold 0
        if (t == 0) partial[g] = sum;
    }
}

template <typename T, int F>
__global__ __launch_bounds__(kThreads) void quantize_tail_kernel(
    const T *__restrict__ w, int64_t n, int64_t g, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, uint8_t *__restrict__ absmax_q, float *__restrict__ absmax_scale,
    float *__restrict__ partial, CodeLut lut) {
    quantize_tail<T, F>(w, n, g, codes, absmax, absmax_q, absmax_scale, partial, lut);
}

// Standalone double quantization: one workgroup per group of 256 c1 values.
__global__ __launch_bounds__(kThreads) void double_quantize_kernel(
    const float *__restrict__ absmax, int64_t nblocks, uint8_t *__restrict__ absmax_q,
    float *__restrict__ absmax_scale) {
    __shared__ float s_red[4];
    const int t = threadIdx.x;
    const int64_t g = blockIdx.x;
    const int64_t b = g * kDqBlock + t;
    const float c1 = (b < nblocks) ? absmax[b] : 0.0f;
    const float c2 = wg_max(fabsf(c1), s_red);
    if (b < nblocks) absmax_q[b] = (uint8_t)dq_encode<kFmtE4M3, true>(c1, c2);
    if (t == 0) absmax_scale[g] = c2;
}

// Threads per group workgroup.
constexpr int kGroupThreads = 512;

// B1 = 64 (and, with double quantization, B2 = 256 without the mean
// offset): the fused group kernel, 8-bit codes in format F, one kernel per
// codebook kind.
template <typename T, int F>
hipError_t launch_quantize_t(const T *w, int64_t n, uint8_t *codes, float *absmax,
                             uint8_t *absmax_q, float *absmax_scale, const CodeLut &lut,
                             hipStream_t s, float *partial = nullptr) {
    const int64_t full = n / kGroup;
    constexpr int TH = kGroupThreads;
    if (full > 0) {
        with_cb<T>(lut, [&](auto cbc) {
            constexpr int CB = decltype(cbc)::value;
            if (absmax_q)
                quantize_groups_kernel<T, true, TH, F, CB><<<dim3((unsigned)full), dim3(TH), 0, s>>>(
                    w, codes, absmax, absmax_q, absmax_scale, nullptr, lut);
            else
                quantize_groups_kernel<T, false, TH, kFmtE4M3, CB><<<dim3((unsigned)full), dim3(TH), 0, s>>>(
                    w, codes, absmax, nullptr, nullptr, partial, lut);
            return hipSuccess;
        });
    }
    if (n % kGroup)
        quantize_tail_kernel<T, F><<<1, kThreads, 0, s>>>(w, n, full, codes, absmax, absmax_q,
                                                          absmax_scale, partial, lut);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_quantize_fmt(const T *w, int64_t n, uint8_t *codes, float *absmax,
                               uint8_t *absmax_q, float *absmax_scale, int fmt, const CodeLut &lut,
                               hipStream_t s) {
    if (fmt == kFmtE5M2)
        return launch_quantize_t<T, kFmtE5M2>(w, n, codes, absmax, absmax_q, absmax_scale, lut, s);
    if (fmt == kFmtLin8)
        return launch_quantize_t<T, kFmtLin8>(w, n, codes, absmax, absmax_q, absmax_scale, lut, s);
    return launch_quantize_t<T, kFmtE4M3>(w, n, codes, absmax, absmax_q, absmax_scale, lut, s);
}

// ---- batched quantization: the tensors of a model in few launches ----

// Entries per launch: their pointers travel in the kernel-argument block.
constexpr int kBatch = 32;

// Up to kBatch tensors of one launch. Workgroup i works on entry k, the last
// with first[k] <= i, at local index i - first[k]; entries past the batch
// hold first = UINT32_MAX. For the tail launch, entry k is workgroup k and
// first[k] is the index of the entry's partial group.
struct QuantBatch {
    const void *w[kBatch];
    uint8_t *codes[kBatch];
    float *absmax[kBatch];
    uint8_t *q[kBatch];
    float *sc[kBatch];
    int64_t n[kBatch];
    uint32_t first[kBatch];
};

__device__ __forceinline__ int batch_entry(const QuantBatch &b, uint32_t wg) {
    int k = 0;
#pragma unroll
    for (int j = 1; j < kBatch; ++j) k = (wg >= b.first[j]) ? j : k;
    return k;
}

// Full groups of every entry: one workgroup per group, as the group kernel.
template <typename T, bool kDQ, int CB>
__global__ __launch_bounds__(kGroupThreads) void quantize_batch_kernel(QuantBatch b, CodeLut lut) {
    const uint32_t wg = blockIdx.x;
    const int k = batch_entry(b, wg);
    quantize_group<T, kDQ, kGroupThreads, kFmtE4M3, CB>(static_cast<const T *>(b.w[k]), b.codes[k],
                                                    b.absmax[k], b.q[k], b.sc[k], nullptr, lut,
                                                    (int64_t)(wg - b.first[k]));
}

// The partial last group of each entry: workgroup k takes entry k's.
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_batch_tail_kernel(QuantBatch b, CodeLut lut) {
    const int k = blockIdx.x;
    quantize_tail<T, kFmtE4M3>(static_cast<const T *>(b.w[k]), b.n[k], (int64_t)b.first[k],
                               b.codes[k], b.absmax[k], b.q[k], b.sc[k], nullptr, lut);
}

// Collects entries into QuantBatch blocks and launches each when full.
// `tail` selects what a launch covers: the full groups of its entries, or
// their partial last groups.
template <typename T>
struct BatchLauncher {
    QuantBatch b;
    int count = 0;
    uint32_t wgs = 0;
    bool tail, dq;
    const CodeLut &lut;
    hipStream_t s;
    hipError_t err = hipSuccess;

    BatchLauncher(bool tail_, bool dq_, const CodeLut &l, hipStream_t st)
        : tail(tail_), dq(dq_), lut(l), s(st) {}

    void flush() {
        if (count == 0) return;
        for (int j = count; j < kBatch; ++j) {
            b.w[j] = nullptr;
            b.codes[j] = nullptr;
            b.absmax[j] = nullptr;
            b.q[j] = nullptr;
            b.sc[j] = nullptr;
            b.n[j] = 0;
            b.first[j] = UINT32_MAX;
        }
        if (tail)
            quantize_batch_tail_kernel<T><<<dim3((unsigned)count), dim3(kThreads), 0, s>>>(b, lut);
        else
            with_cb<T>(lut, [&](auto cbc) {
                constexpr int CB = decltype(cbc)::value;
                if (dq)
                    quantize_batch_kernel<T, true, CB><<<dim3(wgs), dim3(kGroupThreads), 0, s>>>(b, lut);
                else
                    quantize_batch_kernel<T, false, CB><<<dim3(wgs), dim3(kGroupThreads), 0, s>>>(b, lut);
                return hipSuccess;
            });
        const hipError_t e = hipGetLastError();
        if (err == hipSuccess) err = e;
        count = 0;
        wgs = 0;
    }

    // Adds entry e: `units` workgroups (full groups), or its partial group.
    void add(const nf4_batch_entry &e, int64_t units) {
        // a full-group launch stays below 2^31 threads
        constexpr int64_t kMaxWgs = (int64_t(1) << 31) / kGroupThreads;
        if (count == kBatch || (!tail && (int64_t)wgs + units > kMaxWgs)) flush();
        b.w[count] = e.w;
        b.codes[count] = e.codes;
        b.absmax[count] = e.absmax;
        b.q[count] = dq ? e.absmax_q : nullptr;
        b.sc[count] = dq ? e.absmax_scale : nullptr;
        b.n[count] = e.n;
        b.first[count] = tail ? (uint32_t)(e.n / kGroup) : wgs;
        wgs += tail ? 1u : (uint32_t)units;
        ++count;
    }
};

template <typename T>
hipError_t launch_quantize_batched_t(const nf4_batch_entry *e, int32_t count, const CodeLut &lut,
                                     hipStream_t s) {
    hipError_t err = hipSuccess;
    for (int dq = 1; dq >= 0; --dq) {
        BatchLauncher<T> full(false, dq != 0, lut, s), tail(true, dq != 0, lut, s);
        for (int32_t i = 0; i < count; ++i) {
            if ((e[i].absmax_q != nullptr) != (dq != 0) || e[i].n <= 0) continue;
            const int64_t groups = e[i].n / kGroup;
            if (groups > 0) full.add(e[i], groups);
            if (e[i].n % kGroup) tail.add(e[i], 1);
        }
        full.flush();
        tail.flush();
        if (err == hipSuccess) err = full.err != hipSuccess ? full.err : tail.err;
    }
    return err;
}

// ---- storage-format variants: block sizes other than 64, the mean offset ----

// Blockwise quantization with block size B1 (codes and fp32 absmax; double
// quantization follows in its own kernel). A wave works on units of
// U = max(B1, 64 E) weights: one block, or 64 E / B1 whole blocks. Each lane
// holds S = U / (64 E) slices of a unit, slice i at i * 64 + lane, so every
// wave load is one contiguous 1 KiB run as in the group kernel. A block's
// absmax is a DPP max over its B1 / E lanes, or a whole-wave max.
template <typename T, int B1, int CB>
__global__ __launch_bounds__(kThreads) void quantize_blocks_kernel(
    const T *__restrict__ w, int64_t nunits, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, CodeLut lut) {
    using Sl = Slice<T>;
    constexpr int E = Sl::kElems;
    constexpr int U = B1 > 64 * E ? B1 : 64 * E;  // weights per unit
    constexpr int S = U / (64 * E);                // slices per lane and unit
    constexpr int UPW = S >= 4 ? 1 : 4 / S;        // units per wave
    constexpr int LPB = B1 / E;                    // lanes per block (S == 1)
    constexpr int kTab = E * kLutEntries;
    __shared__ float2 s_lut[kTab];

    const int t = threadIdx.x, lane = t & 63;
    const int64_t unit0 = ((int64_t)blockIdx.x * (kThreads / 64) +
                           __builtin_amdgcn_readfirstlane(t >> 6)) * UPW;
    // all loads first (a unit past the end reloads the last one and stores nothing)
    typename Sl::Vec v[UPW][S];
#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const int64_t unit = min(unit0 + u, nunits - 1);
        const typename Sl::Vec *src = reinterpret_cast<const typename Sl::Vec *>(w + unit * U);
#pragma unroll
        for (int i = 0; i < S; ++i) v[u][i] = __builtin_nontemporal_load(&src[i * 64 + lane]);
    }
    for (int i = t; i < kTab; i += kThreads) s_lut[i] = lut_copy_entry(lut.e[i % kLutEntries], i);
    __syncthreads();

#pragma unroll
    for (int u = 0; u < UPW; ++u) {
        const int64_t unit = unit0 + u;
        if (unit >= nunits) break;  // uniform over the wave
        float f[S][E];
        float mf = 0.0f;
#pragma unroll
        for (int i = 0; i < S; ++i) {
            Sl::widen(v[u][i], f[i]);
#pragma unroll
            for (int e = 0; e < E; ++e) mf = fmaxf(mf, fabsf(f[i][e]));
        }
        float m;
        if constexpr (U == B1) {
            m = wave_max_nonneg(mf);
            if (lane == 0) absmax[unit] = m;
        } else {
            uint32_t mb = __float_as_uint(mf);
            mb = dpp_umax<0xB1>(mb);                           // quad_perm [1,0,3,2]
            if (LPB >= 4) mb = dpp_umax<0x4E>(mb);             // quad_perm [2,3,0,1]
            if (LPB >= 8) mb = dpp_umax<0x141>(mb);            // row_half_mirror
            if (LPB >= 16) mb = dpp_umax<0x140>(mb);           // row_mirror
            if (LPB >= 32) mb = max(mb, (uint32_t)__shfl_xor((int)mb, 16));
            m = __uint_as_float(mb);
            if ((lane % LPB) == 0) absmax[unit * (U / B1) + lane / LPB] = m;
        }
#pragma unroll
        for (int i = 0; i < S; ++i) {
            const uint32_t packed = slice_codes_cb<E, CB>(f[i], m, s_lut);
            const int64_t slice = unit * (U / E) + i * 64 + lane;
            if (E == 8)
                reinterpret_cast<uint32_t *>(codes)[slice] = packed;
            else
                reinterpret_cast<uint16_t *>(codes)[slice] = (uint16_t)packed;
        }
    }
}

// The blocks after the last full unit: one thread per block, element by
// element with the correctly rounded division.
template <typename T>
__global__ __launch_bounds__(64) void quantize_blocks_tail_kernel(
    const T *__restrict__ w, int64_t n, int64_t b0, int64_t nblocks, int32_t bs,
    uint8_t *__restrict__ codes, float *__restrict__ absmax, CodeLut lut) {
    __shared__ float2 s_lut[kLutEntries];
    load_lut(lut, s_lut);
    __syncthreads();
    const int64_t b = b0 + (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (b >= nblocks) return;
    const int64_t lo = b * bs;
    const int64_t hi = min(lo + bs, n);
    auto elem = [&](int64_t i) -> float {
        if constexpr (sizeof(T) == 2) return __uint_as_float((uint32_t)w[i] << 16);
        else return w[i];
    };
    float c1 = 0.0f;
    for (int64_t i = lo; i < hi; ++i) c1 = fmaxf(c1, fabsf(elem(i)));
    absmax[b] = c1;
    for (int64_t i = lo; i < hi; i += 2) {
        uint32_t byte = 0;
        for (int j = 0; j < 2 && i + j < hi; ++j) {
            const uint32_t code = exact_code(s_lut, (c1 > 0.0f) ? elem(i + j) / c1 : 0.0f, lut.signmag != 0);
            byte |= code << (4 * j);
        }
        codes[i / 2] = (uint8_t)byte;
    }
}

// Pairwise fp32 sum of an aligned chunk of 4096 values (zeros past n), the
// subtree of the sum over the whole array padded to a power of two: each
// thread adds its 16 values as a tree, then lanes pair up by XOR shuffles
// (x + y == y + x, so both lanes of a pair hold the same node) and the four
// wave sums pair up last. final_mean: one workgroup, writes sum / nf.
constexpr int kSumChunk = 4096;
// The chunk [base, base + 4096) of x (zeros past n), summed pairwise by a
// 256-thread workgroup; every thread gets the sum.
__device__ __forceinline__ float chunk_pairwise_sum(const float *__restrict__ x, int64_t n,
                                                    int64_t base, float *s_w) {
    const int t = threadIdx.x;
    const int64_t b0 = base + 16 * t;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = (b0 + i < n) ? x[b0 + i] : 0.0f;
#pragma unroll
    for (int h = 1; h < 16; h *= 2)
#pragma unroll
        for (int i = 0; i < 16; i += 2 * h) v[i] = v[i] + v[i + h];
    float sum = v[0];
#pragma unroll
    for (int k = 1; k < 64; k *= 2) sum = sum + __shfl_xor(sum, k);
    if ((t & 63) == 0) s_w[t >> 6] = sum;
    __syncthreads();
    return (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
}

__global__ __launch_bounds__(kThreads) void pairwise_sum_kernel(const float *__restrict__ x,
                                                                int64_t n, float *__restrict__ out) {
    __shared__ float s_w[kThreads / 64];
    const float tot = chunk_pairwise_sum(x, n, (int64_t)blockIdx.x * kSumChunk, s_w);
    if (threadIdx.x == 0) out[blockIdx.x] = tot;
}

// Double quantization with group size 2^lb2 in format F (kS: mean offset,
// signed codes). A group of 64 or more blocks is one wave's; smaller groups
// are aligned lane segments of a wave of 64 consecutive blocks. With the
// mean offset every workgroup first finishes the pairwise sum itself from
// the top level's nparts <= 4096 partial sums (the same value everywhere),
// mu = sum / nf, and workgroup 0 stores mu.
template <int F, bool kS>
__global__ __launch_bounds__(kThreads) void dq_generic_kernel(
    const float *__restrict__ absmax, int64_t nblocks, int lb2, const float *__restrict__ parts,
    int64_t nparts, float nf, float *__restrict__ mu_out, uint8_t *__restrict__ q,
    float *__restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) +
                         __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int b2 = 1 << lb2;
    // The first 256 block scales of the wave's group (or its 64 blocks) are
    // loaded before mu is summed, so the two load chains overlap; a larger
    // group reads the rest in its loops.
    constexpr int kCache = 4;
    const int64_t g = wave;
    const int64_t b0 = b2 >= 64 ? (g << lb2) : wave * 64;
    float c[kCache];
#pragma unroll
    for (int i = 0; i < kCache; ++i) {
        const int j = lane + 64 * i;
        const bool in = (b2 >= 64 ? j < b2 : i == 0) && b0 + j < nblocks;
        c[i] = in ? absmax[b0 + j] : 0.0f;
    }
    float mu = 0.0f;
    if constexpr (kS) {
        __shared__ float s_w[kThreads / 64];
        mu = chunk_pairwise_sum(parts, nparts, 0, s_w) / nf;
        if (blockIdx.x == 0 && threadIdx.x == 0) *mu_out = mu;
    }
    auto xof = [&](float cv) -> float { return kS ? cv - mu : cv; };
    auto xval = [&](int j) -> float {  // block b0 + j (j < b2, in range)
        return j < 64 * kCache ? xof(c[j / 64]) : xof(absmax[b0 + j]);
    };
    if (b2 >= 64) {
        if (g >= ((nblocks + b2 - 1) >> lb2)) return;  // uniform over the wave
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kCache; ++i) {
            const int j = lane + 64 * i;
            if (j < b2 && b0 + j < nblocks) m = fmaxf(m, fabsf(xof(c[i])));
        }
        for (int j = lane + 64 * kCache; j < b2; j += 64)
            if (b0 + j < nblocks) m = fmaxf(m, fabsf(xof(absmax[b0 + j])));
        float sc = wave_max_nonneg(m);
        if (F == kFmtLin8) sc = sc / lin_levels<kS>();
        if (lane == 0) scale[g] = sc;
#pragma unroll
        for (int i = 0; i < kCache; ++i) {
            const int j = lane + 64 * i;
            if (j < b2 && b0 + j < nblocks) q[b0 + j] = (uint8_t)dq_encode<F, kS>(xof(c[i]), sc);
        }
        for (int j = lane + 64 * kCache; j < b2; j += 64)
            if (b0 + j < nblocks) q[b0 + j] = (uint8_t)dq_encode<F, kS>(xval(j), sc);
    } else {
        const int64_t b = b0 + lane;
        const bool live = b < nblocks;
        const float x = live ? xof(c[0]) : 0.0f;
        uint32_t mb = __float_as_uint(fabsf(x));
        for (int k = 1; k < b2; k *= 2) mb = max(mb, (uint32_t)__shfl_xor((int)mb, k));
        float sc = __uint_as_float(mb);
        if (F == kFmtLin8) sc = sc / lin_levels<kS>();
        if (live) {
            q[b] = (uint8_t)dq_encode<F, kS>(x, sc);
            if ((lane & (b2 - 1)) == 0) scale[b >> lb2] = sc;
        }
    }
}

template <typename T, int B1>
hipError_t launch_blocks(const T *w, int64_t n, uint8_t *codes, float *absmax, const CodeLut &lut,
                         hipStream_t s) {
    constexpr int E = Slice<T>::kElems;
    constexpr int U = B1 > 64 * E ? B1 : 64 * E;
    constexpr int S = U / (64 * E);
    constexpr int UPW = S >= 4 ? 1 : 4 / S;
    const int64_t nunits = n / U;
    if (nunits > 0) {
        const int64_t waves = (nunits + UPW - 1) / UPW;
        const int64_t wgs = (waves + 3) / 4;
        with_cb<T>(lut, [&](auto cbc) {
            quantize_blocks_kernel<T, B1, decltype(cbc)::value><<<dim3((unsigned)wgs), dim3(kThreads), 0, s>>>(
                w, nunits, codes, absmax, lut);
            return hipSuccess;
        });
    }
    const int64_t nb = (n + B1 - 1) / B1;
    const int64_t b0 = nunits * (U / B1);
    if (b0 < nb)
        quantize_blocks_tail_kernel<T><<<dim3((unsigned)((nb - b0 + 63) / 64)), dim3(64), 0, s>>>(
            w, n, b0, nb, B1, codes, absmax, lut);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_blocks_bs(const T *w, int64_t n, int32_t bs, uint8_t *codes, float *absmax,
                            const CodeLut &lut, hipStream_t s) {
    switch (bs) {
        case 16: return launch_blocks<T, 16>(w, n, codes, absmax, lut, s);
        case 32: return launch_blocks<T, 32>(w, n, codes, absmax, lut, s);
        case 64: return launch_quantize_t<T, kFmtE4M3>(w, n, codes, absmax, nullptr, nullptr, lut, s);
        case 128: return launch_blocks<T, 128>(w, n, codes, absmax, lut, s);
        case 256: return launch_blocks<T, 256>(w, n, codes, absmax, lut, s);
        case 512: return launch_blocks<T, 512>(w, n, codes, absmax, lut, s);
        case 1024: return launch_blocks<T, 1024>(w, n, codes, absmax, lut, s);
        case 2048: return launch_blocks<T, 2048>(w, n, codes, absmax, lut, s);
        default: return launch_blocks<T, 4096>(w, n, codes, absmax, lut, s);
    }
}

int ilog2(int64_t v) {
    int l = 0;
    while ((int64_t(1) << l) < v) ++l;
    return l;
}

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

template <int F, bool kS>
void launch_dq_generic(const float *absmax, int64_t nb, int lb2, const float *parts,
                       int64_t nparts, float *mu, uint8_t *q, float *scale, hipStream_t s) {
    const int64_t waves = lb2 >= 6 ? ((nb + (int64_t(1) << lb2) - 1) >> lb2) : (nb + 63) / 64;
    dq_generic_kernel<F, kS><<<dim3((unsigned)((waves + 3) / 4)), dim3(kThreads), 0, s>>>(
        absmax, nb, lb2, parts, nparts, (float)nb, mu, q, scale);
}

// ---- merging the adapter into the quantized base ----
//
// W_new = quantize(fl32(W' + fl32(s * fl32(d)))), d[n][k] = sum_j A[k][j] B[j][n],
// W' the dequantized base [N x K]. A workgroup owns 64 weight rows and walks a
// run of 256-column tiles; in each tile wave w owns the 64-column block
// kb = k0 + 64 w of the 64 rows. B^T for the 64 rows is transposed into LDS
// once. Per tile and wave:
//   - the delta D[n][k] = sum_j B^T[n][j] A[k][j] on the matrix cores
//     (v_mfma_f32_16x16x32_bf16; A's rows hold the rank index contiguously,
//     so its fragments come straight from memory);
//   - two passes of 32 rows: the delta rows go through LDS so that lane l
//     holds half h = l & 1 of row l / 2's block (32 weights, one 16-byte code
//     load); the lane dequantizes them, adds s * d, the block max is the max
//     of the lane pair, and the merged values get their codes from the same
//     nearest-level search as the quantize kernels.
// The next tile's codes and scales are loaded while the current tile is
// computed; the A fragments are loaded at their use (L2 hits: A is shared by
// every workgroup), which keeps the kernel within 168 VGPRs, three waves per
// SIMD. Waves never wait for each other inside the loop. The new fp32 block
// scales go to absmax (or the workspace) for double quantization.
typedef __bf16 mbf16x8_t __attribute__((ext_vector_type(8)));
typedef float mf32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMergeRows = 64;
constexpr int kMergeCols = 256;
constexpr int kMergeRankMax = 256;
constexpr int kCStride = 68;  // fp32 row stride of a delta tile (rows 4 apart hit other banks)

struct MergeParams {
    const uint8_t *codes;  // base codes
    const uint8_t *q8;     // base E4M3 scale codes, or nullptr
    const float *c2;       // base second-level scales
    const float *absmax;   // base fp32 block scales (when q8 == nullptr)
    const uint16_t *a;     // bf16 [K x r]
    const uint16_t *b;     // bf16 [r x N]
    int64_t n_rows, k_cols;
    int32_t col_tiles, tiles_per_wg, chunks;
    int32_t r, rp;         // rank, and the rank rounded up to 32
    float s;
    uint8_t *new_codes;
    float *new_absmax;
    float lv[16];
};

// Global data of one tile for one lane: A fragments of the first two rank
// steps, and for each 32-row pass the lane's 16 code bytes and block scale.
struct MergeTile {
    u32x4 code[2];
    float c1o[2];
};

// (three waves per SIMD: the register budget fits 168 VGPRs, so three workgroups
// share a CU when their LDS does)
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3))) void merge_requantize_kernel(
    MergeParams p, CodeLut lut) {
    constexpr int kTab = 8 * kLutEntries;
    extern __shared__ __attribute__((aligned(16))) uint16_t s_bt[];  // [64][rp + 8]
    __shared__ __attribute__((aligned(16))) float s_c[4][32 * kCStride];
    __shared__ float2 s_lut[kTab];
    __shared__ float s_lv[16];

    const int t = threadIdx.x, lane = t & 63;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int lr = lane & 15, g = lane >> 4, h = lane & 1;
    const int64_t rt = blockIdx.x / p.chunks;
    const int ct0 = (int)(blockIdx.x % p.chunks) * p.tiles_per_wg;
    const int ct1 = min(ct0 + p.tiles_per_wg, p.col_tiles);
    const int64_t n0 = rt * kMergeRows;
    const int bts = p.rp + 8;

    auto load_tile = [&](int ct) {
        MergeTile d;
        const int64_t kb = (int64_t)ct * kMergeCols + 64 * w;
        const bool live = kb < p.k_cols;  // uniform over the wave
        const int64_t kl = live ? kb : 0;
#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            const int64_t n = n0 + 32 * ps + (lane >> 1);
            const int64_t nl = n < p.n_rows ? n : 0;  // rows past N reload row 0, store nothing
            d.code[ps] = *reinterpret_cast<const u32x4 *>(p.codes + nl * (p.k_cols / 2) + kl / 2 + 16 * h);
            const int64_t ob = nl * (p.k_cols / kBlock) + kl / kBlock;
            d.c1o[ps] = p.q8 ? __builtin_amdgcn_cvt_f32_fp8((int)p.q8[ob], 0) * p.c2[ob / kDqBlock]
                             : p.absmax[ob];
        }
        return d;
    };

    MergeTile cur = load_tile(ct0);

    // B^T tile: Bt[n][j] = B[j][n0 + n], zero past N and past the rank
    // (16 loads per thread in flight, then 16 stores; one pass for r <= 64)
    for (int base = 0; base < kMergeRows * p.rp; base += 16 * kThreads) {
        uint16_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = base + u * kThreads + t;
            const int nn = idx & 63, j = idx >> 6;
            v[u] = (j < p.r && n0 + nn < p.n_rows) ? p.b[(int64_t)j * p.n_rows + n0 + nn] : (uint16_t)0;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int idx = base + u * kThreads + t;
            if (idx < kMergeRows * p.rp) s_bt[(idx & 63) * bts + (idx >> 6)] = v[u];
        }
    }
    for (int i = t; i < kTab; i += kThreads) s_lut[i] = lut_copy_entry(lut.e[i % kLutEntries], i);
    if (t < 16) s_lv[t] = p.lv[t];
    __syncthreads();

    float *cw = s_c[w];
    for (int ct = ct0; ct < ct1; ++ct) {
        const MergeTile nxt = load_tile(min(ct + 1, ct1 - 1));
        const int64_t kb = (int64_t)ct * kMergeCols + 64 * w;
        if (kb >= p.k_cols) continue;  // uniform over the wave

        // the delta of the wave's block: D[16 tn + 4 g + q][16 tk + lr] in acc[tn][tk][q]
        mf32x4_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mf32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int js = 0; js < p.rp / 32; ++js) {
            const int j0 = 32 * js + 8 * g;
            u32x4 bq[4], ao[4];
#pragma unroll
            for (int tk = 0; tk < 4; ++tk) {
                    bq[tk] = j0 < p.r
                                 ? *reinterpret_cast<const u32x4 *>(p.a + (kb + 16 * tk + lr) * p.r + j0)
                                 : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                ao[tn] = *reinterpret_cast<const u32x4 *>(s_bt + (16 * tn + lr) * bts + j0);
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                for (int tk = 0; tk < 4; ++tk)
                    acc[tn][tk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(mbf16x8_t, ao[tn]), __builtin_bit_cast(mbf16x8_t, bq[tk]),
                        acc[tn][tk], 0, 0, 0);
        }

#pragma unroll
        for (int ps = 0; ps < 2; ++ps) {
            // rows 32 ps .. +31 of the delta into the wave's LDS tile (a wave's
            // LDS accesses complete in order, so no barrier is needed between
            // its writes, its reads and the next pass's writes)
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
#pragma unroll
                for (int tk = 0; tk < 4; ++tk)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        cw[(16 * tn + 4 * g + q) * kCStride + 16 * tk + lr] = acc[2 * ps + tn][tk][q];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

            const int64_t n = n0 + 32 * ps + (lane >> 1);
            const float *crow = cw + (lane >> 1) * kCStride + 32 * h;
            const u32x4 oc = cur.code[ps];
            const uint32_t dw[4] = {oc.x, oc.y, oc.z, oc.w};
            const float c1o = cur.c1o[ps];
            float wm[4][8];
            float m = 0.0f;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const f32x4 da = *reinterpret_cast<const f32x4 *>(crow + 8 * d);
                const f32x4 db = *reinterpret_cast<const f32x4 *>(crow + 8 * d + 4);
                const float dl[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float wold = s_lv[(dw[d] >> (4 * e)) & 15u] * c1o;
                    const float delta = p.s * dl[e];
                    wm[d][e] = wold + delta;
                    m = fmaxf(m, fabsf(wm[d][e]));
                }
            }
            m = __uint_as_float(dpp_umax<0xB1>(__float_as_uint(m)));  // the lane pair's max
            uint32_t packed[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) packed[d] = slice_codes<8>(wm[d], m, s_lut);
            if (n < p.n_rows) {
                *reinterpret_cast<u32x4 *>(p.new_codes + n * (p.k_cols / 2) + kb / 2 + 16 * h) =
                    u32x4{packed[0], packed[1], packed[2], packed[3]};
                if (h == 0) p.new_absmax[n * (p.k_cols / kBlock) + kb / kBlock] = m;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        cur = nxt;
    }
}

}  // namespace

hipError_t launch_quantize(const void *w, nf4_dtype dt, int64_t n, uint8_t *codes, float *absmax,
                           uint8_t *absmax_q, float *absmax_scale, hipStream_t s) {
    if (dt == NF4_BF16)
        return launch_quantize_t<uint16_t, kFmtE4M3>(static_cast<const uint16_t *>(w), n, codes,
                                                     absmax, absmax_q, absmax_scale, *code_lut(), s);
    return launch_quantize_t<float, kFmtE4M3>(static_cast<const float *>(w), n, codes, absmax,
                                              absmax_q, absmax_scale, *code_lut(), s);
}

hipError_t launch_quantize_batched(const nf4_batch_entry *e, int32_t count, nf4_dtype dt,
                                   hipStream_t s) {
    if (dt == NF4_BF16) return launch_quantize_batched_t<uint16_t>(e, count, *code_lut(), s);
    return launch_quantize_batched_t<float>(e, count, *code_lut(), s);
}

hipError_t launch_double_quantize(const float *absmax, int64_t nblocks, uint8_t *absmax_q,
                                  float *absmax_scale, hipStream_t s) {
    const int64_t groups = (nblocks + kDqBlock - 1) / kDqBlock;
    double_quantize_kernel<<<dim3((unsigned)groups), dim3(kThreads), 0, s>>>(absmax, nblocks,
                                                                             absmax_q, absmax_scale);
    return hipGetLastError();
}


size_t double_quantize_ex_workspace(int64_t nblocks, const nf4_format &f) {
    if (!f.dq_mean_offset) return 0;
    const int64_t l1 = std::max<int64_t>(1, (nblocks + kSumChunk - 1) / kSumChunk);
    const int64_t l2 = std::max<int64_t>(1, (l1 + kSumChunk - 1) / kSumChunk);
    return round256(4 * (size_t)l1) + round256(4 * (size_t)l2);
}

// Two-pass layout: fp32 block scales, then (mean offset, B1 = 64) the
// pairwise sums of the 256-block groups, then the partial-sum levels.
size_t quantize_ex_workspace(int64_t n, const nf4_format &f) {
    const int64_t nb = (n + f.blocksize - 1) / f.blocksize;
    const bool fused = f.blocksize == kBlock && f.dq_blocksize == kDqBlock && !f.dq_mean_offset;
    if (fused) return 0;
    const size_t groups = f.dq_mean_offset ? round256(4 * (size_t)((nb + kDqBlock - 1) / kDqBlock)) : 0;
    return round256(4 * (size_t)nb) + groups + double_quantize_ex_workspace(nb, f);
}

// parts / nparts: partial sums that already cover aligned power-of-two runs
// of the block scales (the group sums of the quantize kernel), or nullptr to
// start from the block scales themselves.
hipError_t launch_double_quantize_ex(const float *absmax, int64_t nb, const nf4_format &f,
                                     uint8_t *absmax_q, float *absmax_scale,
                                     float *absmax_offset, void *workspace, hipStream_t s,
                                     const float *parts, int64_t nparts) {
    const int lb2 = ilog2(f.dq_blocksize);
    if (f.dq_mean_offset) {
        // mu: the pairwise sum level by level (ping-pong between two partial
        // buffers) down to one chunk, which the DQ kernel finishes itself
        const int64_t l1 = std::max<int64_t>(1, (nb + kSumChunk - 1) / kSumChunk);
        float *buf[2] = {static_cast<float *>(workspace),
                         static_cast<float *>(workspace) + round256(4 * (size_t)l1) / 4};
        const float *src = parts ? parts : absmax;
        int64_t len = parts ? nparts : nb;
        for (int lvl = 0; len > kSumChunk; ++lvl) {
            const int64_t outlen = (len + kSumChunk - 1) / kSumChunk;
            pairwise_sum_kernel<<<dim3((unsigned)outlen), dim3(kThreads), 0, s>>>(src, len, buf[lvl & 1]);
            src = buf[lvl & 1];
            len = outlen;
        }
        switch (f.dq_format) {
            case kFmtE5M2: launch_dq_generic<kFmtE5M2, true>(absmax, nb, lb2, src, len, absmax_offset, absmax_q, absmax_scale, s); break;
            case kFmtLin8: launch_dq_generic<kFmtLin8, true>(absmax, nb, lb2, src, len, absmax_offset, absmax_q, absmax_scale, s); break;
            default: launch_dq_generic<kFmtE4M3, true>(absmax, nb, lb2, src, len, absmax_offset, absmax_q, absmax_scale, s);
        }
    } else {
        switch (f.dq_format) {
            case kFmtE5M2: launch_dq_generic<kFmtE5M2, false>(absmax, nb, lb2, nullptr, 0, nullptr, absmax_q, absmax_scale, s); break;
            case kFmtLin8: launch_dq_generic<kFmtLin8, false>(absmax, nb, lb2, nullptr, 0, nullptr, absmax_q, absmax_scale, s); break;
            default: launch_dq_generic<kFmtE4M3, false>(absmax, nb, lb2, nullptr, 0, nullptr, absmax_q, absmax_scale, s);
        }
    }
    return hipGetLastError();
}

hipError_t launch_quantize_ex(const void *w, nf4_dtype dt, int64_t n, const nf4_format &f,
                              uint8_t *codes, float *absmax, uint8_t *absmax_q,
                              float *absmax_scale, float *absmax_offset, void *workspace,
                              hipStream_t s) {
    const bool dq = absmax_q != nullptr;
    const bool bf = dt == NF4_BF16;
    const CodeLut &lut = *code_lut_for(f.codebook);
    const bool fused = f.blocksize == kBlock &&
                       (!dq || (f.dq_blocksize == kDqBlock && !f.dq_mean_offset));
    if (fused) {
        if (bf)
            return launch_quantize_fmt<uint16_t>(static_cast<const uint16_t *>(w), n, codes,
                                                 absmax, absmax_q, absmax_scale, f.dq_format, lut, s);
        return launch_quantize_fmt<float>(static_cast<const float *>(w), n, codes, absmax,
                                          absmax_q, absmax_scale, f.dq_format, lut, s);
    }
    // two passes: codes and fp32 absmax, then double quantization
    const int64_t nb = (n + f.blocksize - 1) / f.blocksize;
    float *am = absmax;
    char *rest = static_cast<char *>(workspace);
    float *gsum = nullptr;  // group sums of the mean offset (B1 = 64)
    int64_t ngroups = 0;
    if (dq) {
        if (!am) am = static_cast<float *>(workspace);
        rest += round256(4 * (size_t)nb);
        if (f.dq_mean_offset) {
            ngroups = (nb + kDqBlock - 1) / kDqBlock;
            if (f.blocksize == kBlock) gsum = reinterpret_cast<float *>(rest);
            rest += round256(4 * (size_t)ngroups);
        }
    }
    hipError_t e;
    if (gsum)
        e = bf ? launch_quantize_t<uint16_t, kFmtE4M3>(static_cast<const uint16_t *>(w), n, codes, am,
                                                       nullptr, nullptr, lut, s, gsum)
               : launch_quantize_t<float, kFmtE4M3>(static_cast<const float *>(w), n, codes, am,
                                                    nullptr, nullptr, lut, s, gsum);
    else
        e = bf ? launch_blocks_bs<uint16_t>(static_cast<const uint16_t *>(w), n, f.blocksize, codes,
                                            am, lut, s)
               : launch_blocks_bs<float>(static_cast<const float *>(w), n, f.blocksize, codes, am,
                                         lut, s);
    if (e != hipSuccess || !dq) return e;
    return launch_double_quantize_ex(am, nb, f, absmax_q, absmax_scale, absmax_offset, rest, s,
                                     gsum, ngroups);
}


size_t merge_workspace(int64_t n_out, int64_t k_in) {
    return round256(4 * (size_t)(n_out * (k_in / kBlock)));
}

hipError_t launch_merge(const nf4_weight &w, const uint16_t *a, const uint16_t *b, int32_t r,
                        float s_lora, uint8_t *codes_out, float *absmax_out, uint8_t *absmax_q_out,
                        float *absmax_scale_out, void *workspace, hipStream_t s) {
    MergeParams p;
    p.codes = w.codes;
    p.q8 = w.absmax_q;
    p.c2 = w.absmax_scale;
    p.absmax = w.absmax;
    p.a = a;
    p.b = b;
    p.n_rows = w.n_out;
    p.k_cols = w.k_in;
    p.col_tiles = (int32_t)((w.k_in + kMergeCols - 1) / kMergeCols);
    p.r = r;
    p.rp = (r + 31) / 32 * 32;
    p.s = s_lora;
    p.new_codes = codes_out;
    p.new_absmax = absmax_out ? absmax_out : static_cast<float *>(workspace);
    for (int i = 0; i < 16; ++i) p.lv[i] = kLevels[i];
    // as many workgroups as fit the CUs at once (three per CU by registers,
    // fewer when the adapter's LDS tile is large), each walking a run of
    // column tiles
    const size_t lds = (size_t)kMergeRows * (p.rp + 8) * 2;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    hipFuncAttributes fa{};
    size_t static_lds = 0;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void *>(merge_requantize_kernel)) == hipSuccess)
        static_lds = fa.sharedSizeBytes;
    const int64_t per_cu = std::max<int64_t>(1, std::min<int64_t>(3, (int64_t)(160 * 1024) / (int64_t)(lds + static_lds)));
    const int64_t row_tiles = (w.n_out + kMergeRows - 1) / kMergeRows;
    const int64_t target = per_cu * cus;
    int64_t per = (row_tiles * p.col_tiles + target - 1) / target;
    per = std::max<int64_t>(1, std::min<int64_t>(per, p.col_tiles));
    p.tiles_per_wg = (int32_t)per;
    p.chunks = (int32_t)((p.col_tiles + per - 1) / per);
    merge_requantize_kernel<<<dim3((unsigned)(row_tiles * p.chunks)), dim3(kThreads), lds, s>>>(
        p, *code_lut());
    if (absmax_q_out) {
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_double_quantize(p.new_absmax, w.n_out * (w.k_in / kBlock), absmax_q_out,
                                      absmax_scale_out, s);
    }
    return hipGetLastError();
}

}  // namespace nf4
