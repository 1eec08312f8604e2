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
// The nearest level is found without a 16-way search: n is approximated by
// q = fl(w * fl(1/c1)) (one multiply), bucketed (one fma + convert), and the
// code is base + (q >= thr) from a 33-entry LDS table. q differs from the
// exact fl(w / c1) by < 1.8e-7; lanes with q within 2^-20 of a switch point
// redo their slice with the correctly rounded division, so codes are exactly
// those of the definition.
#pragma clang fp contract(off)

#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;

// Max over the whole workgroup of T threads; every thread gets the result.
template <int T = kThreads>
__device__ __forceinline__ float wg_max(float v, float *s_red) {
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) s_red[wave] = v;
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
__device__ __forceinline__ float2 lut_entry(const float2 *s_lut, float v) {
    return *reinterpret_cast<const float2 *>(reinterpret_cast<const char *>(s_lut) + lut_offset(v));
}

// Max of non-negative floats via their bit patterns (monotone as unsigned),
// with the neighbour lane brought in by DPP.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
    return max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xF, 0xF, false));
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

// Codes of one lane's slice. c1 is the block absmax (all lanes of the block
// hold the same value). Returns the packed nibbles, element e at bits 4e.
template <int E>
__device__ __forceinline__ uint32_t slice_codes(const float (&f)[E], float c1, const float2 *s_lut) {
    // rcp ~ 1/c1 from v_rcp_f32 (within 1 ulp for a normal result): then
    // |q - fl(w/c1)| stays below 2.4e-7 for |w| <= c1, well inside kNearTol.
    // Blocks with c1 == 0 (all zero) take rcp = 0 (q = 0 -> code 7). A c1
    // outside [2^-125, 2^125] - whose reciprocal would overflow or fall into
    // the subnormal range, where v_rcp_f32 is not that accurate - takes the
    // exact path for the whole slice.
    const bool in_range = (c1 >= 0x1p-125f) & (c1 <= 0x1p125f);
    const bool outside = (c1 > 0.0f) & !in_range;
    const float rcp = in_range ? __builtin_amdgcn_rcpf(c1) : 0.0f;
    uint32_t packed = 0;
    float dmin = __builtin_inff();
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float q = f[e] * rcp;
        const float2 ent = lut_entry(s_lut, q);
        const float d = q - ent.x;
        const uint32_t code = (uint32_t)__float_as_int(ent.y) + (d >= 0.0f ? 1u : 0u);
        dmin = fminf(dmin, fabsf(d));
        packed |= code << (4 * e);
    }
    if (outside | !(dmin >= kNearTol)) {  // rare: redo with the correctly rounded division
        packed = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float nrm = f[e] / c1;
            const float2 ent = lut_entry(s_lut, nrm);
            const uint32_t code = (uint32_t)__float_as_int(ent.y) + (nrm >= ent.x ? 1u : 0u);
            packed |= code << (4 * e);
        }
    }
    return packed;
}

__device__ __forceinline__ void load_lut(const CodeLut &lut, float2 *s_lut) {
    if (threadIdx.x < kLutEntries)
        s_lut[threadIdx.x] = make_float2(lut.e[threadIdx.x].thr, __int_as_float(lut.e[threadIdx.x].base));
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

    __shared__ float2 s_lut[kLutEntries];
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
    // (every thread stores its entry; the copies are identical)
    s_lut[t % kLutEntries] = make_float2(le.thr, __int_as_float(le.base));
    __syncthreads();

#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
        float f[E];
        S::widen(v[i], f);
        float mf = fabsf(f[0]);
#pragma unroll
        for (int e = 1; e < E; ++e) mf = fmaxf(mf, fabsf(f[e]));
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
            uint32_t code = 7;
            if (c1 > 0.0f) {
                const float nrm = elem(i + j) / c1;
                const float2 ent = lut_entry(s_lut, nrm);
                code = (uint32_t)__float_as_int(ent.y) + (nrm >= ent.x ? 1u : 0u);
            }
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
