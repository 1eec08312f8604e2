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

// Byte offset of the table entry of a normalised value (see CodeLut).
__device__ __forceinline__ uint32_t lut_offset(float v) {
    return lut_offset_bits(fmaf(v, 128.0f, 128.0f + 0x1p23f));
}
__device__ __forceinline__ float2 lut_at(const float2 *s_lut, uint32_t off) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(s_lut) + off);
}
// Code of an exactly normalised value (the definition's fl32(w / c1)).
__device__ __forceinline__ uint32_t exact_code(const float2 *s_lut, float nrm) {
    const float2 ent = lut_at(s_lut, lut_offset(nrm));
    return (uint32_t)__float_as_int(ent.y) - (nrm < ent.x ? 1u : 0u);
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

// Codes of one lane's slice. c1 is the block absmax (all lanes of the block
// hold the same value). s_lut holds E copies of the table, copy e with the
// top code shifted to nibble e. Returns the packed nibbles, element e at
// bits 4e.
template <int E>
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
        const float2 ent = lut_at(s_lut + e * kLutEntries,
                                  lut_offset_bits(fmaf(f[e], rcp128, 128.0f + 0x1p23f)));
        d[e] = fmaf(f[e], rcp, -ent.x);
        top |= __float_as_uint(ent.y);
    }
    float dmin = fabsf(d[0]);
#pragma unroll
    for (int e = 1; e < E; ++e) dmin = fminf(dmin, fabsf(d[e]));
    uint32_t packed = top - sign_nibbles<E>(d);
    if (outside | !(dmin >= kNearTol)) {  // rare: redo with the correctly rounded division
        packed = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) packed |= exact_code(s_lut, f[e] / c1) << (4 * e);
    }
    return packed;
}

// Entry i of the table copies (copy i / kLutEntries, see slice_codes).
__device__ __forceinline__ float2 lut_copy_entry(const LutEntry &le, int i) {
    return make_float2(le.thr, __int_as_float(le.hi << (4 * (i / kLutEntries))));
}

__device__ __forceinline__ void load_lut(const CodeLut &lut, float2 *s_lut) {
    if (threadIdx.x < kLutEntries) s_lut[threadIdx.x] = lut_copy_entry(lut.e[threadIdx.x], 0);
}

// Double quantization of the group's 256 c1 values held in s_c1 (threads
// 0..255 each own one block; a larger workgroup's other threads only join
// the barriers).
template <int T>
__device__ __forceinline__ void group_dq(const float *s_c1, float *s_red, uint32_t *s_q8,
                                         uint8_t *absmax_q, float *absmax_scale, int64_t g) {
    const int t = threadIdx.x;
    const float c1 = (t < kDqBlock) ? s_c1[t] : 0.0f;
    const float c2 = wg_max<T>(c1, s_red);
    if (t < kDqBlock) {
        const float ratio = (c2 > 0.0f) ? c1 / c2 : 0.0f;
        reinterpret_cast<uint8_t *>(s_q8)[t] = (uint8_t)e4m3_encode_unit(ratio);
    }
    __syncthreads();
    if (t < kDqBlock / 4) reinterpret_cast<uint32_t *>(absmax_q + g * kDqBlock)[t] = s_q8[t];
    if (t == 0) absmax_scale[g] = c2;
}

// One workgroup of TH threads per full group of 16384 weights.
template <typename T, bool kDQ, int TH>
__global__ __launch_bounds__(TH) void quantize_groups_kernel(
    const T *__restrict__ w, uint8_t *__restrict__ codes, float *__restrict__ absmax,
    uint8_t *__restrict__ absmax_q, float *__restrict__ absmax_scale, CodeLut lut) {
    using S = Slice<T>;
    constexpr int E = S::kElems;               // weights per lane slice
    constexpr int LPB = kBlock / E;            // lanes per block
    constexpr int SLICES = kGroup / E;         // slices per group
    constexpr int ITERS = SLICES / TH;         // slices per thread
    constexpr int BPI = TH / LPB;              // blocks per iteration

    constexpr int kTab = E * kLutEntries;       // entries of the E table copies
    static_assert(kTab <= TH, "one table entry per thread");
    __shared__ float2 s_lut[kTab];
    __shared__ float s_c1[kDqBlock];
    __shared__ float s_red[TH / 64];
    __shared__ uint32_t s_q8[kDqBlock / 4];

    const int t = threadIdx.x;
    const int64_t g = blockIdx.x;
    const typename S::Vec *src = reinterpret_cast<const typename S::Vec *>(w + g * kGroup);

    // The table comes from the argument block through a vector load: issued
    // first and stored to LDS after the weight loads are on their way, so its
    // wait does not cover them.
    const LutEntry le = lut.e[t % kLutEntries];
    __builtin_amdgcn_sched_barrier(0);
    typename S::Vec v[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) v[i] = __builtin_nontemporal_load(&src[i * TH + t]);
    // (threads past the table store a duplicate of an entry, unconditionally)
    s_lut[t % kTab] = lut_copy_entry(le, t % kTab);
    __syncthreads();

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
        const int blk = i * BPI + t / LPB;  // block within the group
        if ((t % LPB) == 0) {
            if (kDQ) s_c1[blk] = m;
            if (absmax) absmax[g * kDqBlock + blk] = m;
        }
        const uint32_t packed = slice_codes<E>(f, m, s_lut);
        const int64_t slice = (int64_t)g * SLICES + i * TH + t;
        if (E == 8)
            reinterpret_cast<uint32_t *>(codes)[slice] = packed;
        else
            reinterpret_cast<uint16_t *>(codes)[slice] = (uint16_t)packed;
    }
    if (kDQ) {
        __syncthreads();
        group_dq<TH>(s_c1, s_red, s_q8, absmax_q, absmax_scale, g);
    }
}

// The final partial group: thread t owns block t of the group and works
// element by element with guarded accesses.
template <typename T>
__global__ __launch_bounds__(kThreads) void quantize_tail_kernel(
    const T *__restrict__ w, int64_t n, int64_t g, uint8_t *__restrict__ codes,
    float *__restrict__ absmax, uint8_t *__restrict__ absmax_q, float *__restrict__ absmax_scale,
    CodeLut lut) {
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
            const uint32_t code = (c1 > 0.0f) ? exact_code(s_lut, elem(i + j) / c1) : 7u;
            byte |= code << (4 * j);
        }
        codes[i / 2] = (uint8_t)byte;
    }
    if (absmax_q) {
        __syncthreads();
        const float c2 = wg_max(s_c1[t], s_red);
        const int64_t nblocks = (n + kBlock - 1) / kBlock;
        if (b < nblocks) {
            const float ratio = (c2 > 0.0f) ? s_c1[t] / c2 : 0.0f;
            absmax_q[b] = (uint8_t)e4m3_encode_unit(ratio);
        }
        if (t == 0) absmax_scale[g] = c2;
    }
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
    if (b < nblocks) {
        const float ratio = (c2 > 0.0f) ? c1 / c2 : 0.0f;
        absmax_q[b] = (uint8_t)e4m3_encode_unit(ratio);
    }
    if (t == 0) absmax_scale[g] = c2;
}

// Threads per group workgroup.
constexpr int kGroupThreads = 512;

template <typename T>
hipError_t launch_quantize_t(const T *w, int64_t n, uint8_t *codes, float *absmax,
                             uint8_t *absmax_q, float *absmax_scale, hipStream_t s) {
    const CodeLut &lut = *code_lut();
    const int64_t full = n / kGroup;
    constexpr int TH = kGroupThreads;
    if (full > 0) {
        if (absmax_q)
            quantize_groups_kernel<T, true, TH><<<dim3((unsigned)full), dim3(TH), 0, s>>>(
                w, codes, absmax, absmax_q, absmax_scale, lut);
        else
            quantize_groups_kernel<T, false, TH><<<dim3((unsigned)full), dim3(TH), 0, s>>>(
                w, codes, absmax, nullptr, nullptr, lut);
    }
    if (n % kGroup)
        quantize_tail_kernel<T><<<1, kThreads, 0, s>>>(w, n, full, codes, absmax, absmax_q,
                                                       absmax_scale, lut);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void *w, nf4_dtype dt, int64_t n, uint8_t *codes, float *absmax,
                           uint8_t *absmax_q, float *absmax_scale, hipStream_t s) {
    if (dt == NF4_BF16)
        return launch_quantize_t<uint16_t>(static_cast<const uint16_t *>(w), n, codes, absmax,
                                           absmax_q, absmax_scale, s);
    return launch_quantize_t<float>(static_cast<const float *>(w), n, codes, absmax, absmax_q,
                                    absmax_scale, s);
}

hipError_t launch_double_quantize(const float *absmax, int64_t nblocks, uint8_t *absmax_q,
                                  float *absmax_scale, hipStream_t s) {
    const int64_t groups = (nblocks + kDqBlock - 1) / kDqBlock;
    double_quantize_kernel<<<dim3((unsigned)groups), dim3(kThreads), 0, s>>>(absmax, nblocks,
                                                                             absmax_q, absmax_scale);
    return hipGetLastError();
}

}  // namespace nf4
