// dequantize.hip - NF4 dequantization for gfx950 ([MF] "Block-Wise
// Quantization Mechanics", reconstruction; the dequantize(c1^FP8, c2, W^NF4)
// of "Forward Pass Computation"; source key in nf4_internal.h).
//
//   c1'(b) = fl32(decode8(absmax_q[b]) * c2[b / 256])   (or absmax[b] without DQ)
//   w'     = fl32(q[code] * c1'(b)), then nearest-even bf16 for bf16 output.
//
// Work split: a wave owns chunks of 2048 weights (1 KiB of codes, 32 blocks).
// Lane l reads code dwords j*256 + 4l (j = 0..3), so each wave load is 256
// contiguous bytes and each lane's 8 weights per dword are contiguous in the
// output: a bf16 store is one 16-byte vector per lane and 1 KiB per wave.
// A byte of codes is turned into its two levels by one 8-byte LDS read from a
// 256-entry (low, high) level table; the scale multiply and the bf16 rounding
// (v_cvt_pk_bf16_f32) follow.
#pragma clang fp contract(off)

#include "nf4_internal.h"

namespace nf4 {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 2048;             // weights per wave chunk
constexpr int kChunkBytes = kChunk / 2;  // code bytes per chunk

struct Levels {
    float q[16];
};

// Entry e of the table is (q[e & 15], q[e >> 4]). The levels are kernel
// arguments (scalar loads); a select chain copies them to LDS first, so that
// building the table issues no vector-memory load (which would be waited on
// together with the code loads already in flight). Ends with a barrier.
__device__ __forceinline__ void build_pair_table(const Levels &lv, float *s_lv, float2 *s_pair) {
    const int t = threadIdx.x;  // 256 threads: one entry each
    if (t < 16) {
        // (the empty asm keeps each level an opaque scalar, so the chain is
        // not turned back into an indexed load of the argument block)
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float q = lv.q[i];
            asm volatile("" : "+s"(q));
            v = t == i ? q : v;
        }
        s_lv[t] = v;
    }
    __syncthreads();
    s_pair[t] = make_float2(s_lv[t & 15], s_lv[t >> 4]);
    __syncthreads();
}

template <typename O> struct Out;
template <> struct Out<uint16_t> {  // bf16
    __device__ static void store8(uint16_t *dst, const float (&v)[8]) {
        u32x4 o;
        o.x = pack_bf16x2(v[0], v[1]);
        o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]);
        o.w = pack_bf16x2(v[6], v[7]);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4 *>(dst));
    }
    __device__ static void store1(uint16_t *dst, float v) {
        *dst = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
};
template <> struct Out<float> {
    __device__ static void store8(float *dst, const float (&v)[8]) {
        const f32x4 a = {v[0], v[1], v[2], v[3]};
        const f32x4 b = {v[4], v[5], v[6], v[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4 *>(dst));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4 *>(dst + 4));
    }
    __device__ static void store1(float *dst, float v) { *dst = v; }
};

// The chunks of workgroup wg of a tensor with nchunks full chunks.
template <typename O, bool kDQ, int kCPW>
__device__ __forceinline__ void dequantize_chunks(
    const uint8_t *__restrict__ codes, int64_t nchunks, const float *__restrict__ absmax,
    const uint8_t *__restrict__ absmax_q, const float *__restrict__ absmax_scale,
    O *__restrict__ out, Levels lv, const int64_t wg) {
    __shared__ float2 s_pair[256];
    __shared__ float s_lv[16];
    const int lane = threadIdx.x & 63;
    // wave index in scalar registers: the chunk's scale data is then fetched
    // with scalar loads (32 E4M3 codes and one c2 per chunk: a chunk of 32
    // blocks never straddles a group of 256)
    const int64_t wave = wg * (kThreads / 64) +
                         __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // all code loads of the wave's chunks first (a chunk past the end reloads
    // the last one and stores nothing)
    uint32_t d[kCPW][4];
#pragma unroll
    for (int c = 0; c < kCPW; ++c) {
        const int64_t chunk = min(wave * kCPW + c, nchunks - 1);
        const uint32_t *src = reinterpret_cast<const uint32_t *>(codes + chunk * kChunkBytes);
#pragma unroll
        for (int j = 0; j < 4; ++j) d[c][j] = __builtin_nontemporal_load(&src[j * 64 + lane]);
    }
    build_pair_table(lv, s_lv, s_pair);

#pragma unroll
    for (int c = 0; c < kCPW; ++c) {
        const int64_t chunk = wave * kCPW + c;
        if (chunk >= nchunks) return;
        const int64_t blk0 = chunk * (kChunk / kBlock);
        // scale of dword j: block 8 j + lane / 8 of the chunk
        float s[4];
        if constexpr (kDQ) {
            const uint32_t *q32 = reinterpret_cast<const uint32_t *>(absmax_q + blk0);
            const float c2 = absmax_scale[blk0 / kDqBlock];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t code8 = __builtin_amdgcn_perm(q32[2 * j + 1], q32[2 * j], (uint32_t)(lane >> 3));
                // gfx950's fp8 -> f32 convert decodes OCP E4M3FN exactly
                s[j] = __builtin_amdgcn_cvt_f32_fp8((int)code8, 0) * c2;
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] = absmax[blk0 + j * 8 + (lane >> 3)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float2 qq = s_pair[(d[c][j] >> (8 * k)) & 0xFFu];
                v[2 * k] = qq.x * s[j];
                v[2 * k + 1] = qq.y * s[j];
            }
            Out<O>::store8(out + chunk * kChunk + j * 512 + lane * 8, v);
        }
    }
}

template <typename O, bool kDQ, int kCPW>
__global__ __launch_bounds__(kThreads) void dequantize_chunks_kernel(
    const uint8_t *__restrict__ codes, int64_t nchunks, const float *__restrict__ absmax,
    const uint8_t *__restrict__ absmax_q, const float *__restrict__ absmax_scale,
    O *__restrict__ out, Levels lv) {
    dequantize_chunks<O, kDQ, kCPW>(codes, nchunks, absmax, absmax_q, absmax_scale, out, lv,
                                    (int64_t)blockIdx.x);
}

// Weight i of a tensor, one weight per thread (s_pair built).
template <typename O>
__device__ __forceinline__ void dequantize_one(const uint8_t *__restrict__ codes, int64_t i,
                                               const float *__restrict__ absmax,
                                               const uint8_t *__restrict__ absmax_q,
                                               const float *__restrict__ absmax_scale,
                                               O *__restrict__ out, const float2 *s_pair) {
    const uint32_t code = (codes[i >> 1] >> (4 * (i & 1))) & 15u;
    const float c1 = block_scale(i / kBlock, absmax, absmax_q, absmax_scale);
    Out<O>::store1(out + i, s_pair[code].x * c1);
}

// Remaining weights after the last full chunk: one weight per thread.
template <typename O>
__global__ __launch_bounds__(kThreads) void dequantize_tail_kernel(
    const uint8_t *__restrict__ codes, int64_t start, int64_t n, const float *__restrict__ absmax,
    const uint8_t *__restrict__ absmax_q, const float *__restrict__ absmax_scale,
    O *__restrict__ out, Levels lv) {
    __shared__ float2 s_pair[256];
    __shared__ float s_lv[16];
    build_pair_table(lv, s_lv, s_pair);
    const int64_t i = start + (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    dequantize_one<O>(codes, i, absmax, absmax_q, absmax_scale, out, s_pair);
}

// ---- batched dequantization: the tensors of a model in few launches ----

// Entries per launch: their pointers travel in the kernel-argument block.
constexpr int kBatch = 32;
constexpr int kGroupWgs = kGroup / (kChunk * 2 * (kThreads / 64));  // workgroups per group
static_assert(kGroupWgs == 1, "a chunk workgroup covers one DQ group");

// Up to kBatch tensors of one launch. In the chunk launch, workgroup i works
// on entry k, the last with first[k] <= i, at local index i - first[k];
// entries past the batch hold first = UINT32_MAX. In the tail launch,
// workgroup k takes the weights of entry k from index n / 16384 * 16384 on.
struct DequantBatch {
    const uint8_t *codes[kBatch];
    const float *absmax[kBatch];
    const uint8_t *q[kBatch];
    const float *sc[kBatch];
    void *out[kBatch];
    int64_t n[kBatch];
    uint32_t first[kBatch];
};

template <typename O, bool kDQ>
__global__ __launch_bounds__(kThreads) void dequantize_batch_kernel(DequantBatch b, Levels lv) {
    const uint32_t wg = blockIdx.x;
    int k = 0;
#pragma unroll
    for (int j = 1; j < kBatch; ++j) k = (wg >= b.first[j]) ? j : k;
    // every chunk of a full group exists, so nchunks only bounds the loads
    dequantize_chunks<O, kDQ, 2>(b.codes[k], (b.n[k] / kGroup) * (kGroup / kChunk), b.absmax[k],
                                 b.q[k], b.sc[k], static_cast<O *>(b.out[k]), lv,
                                 (int64_t)(wg - b.first[k]));
}

template <typename O>
__global__ __launch_bounds__(kThreads) void dequantize_batch_tail_kernel(DequantBatch b, Levels lv) {
    __shared__ float2 s_pair[256];
    __shared__ float s_lv[16];
    build_pair_table(lv, s_lv, s_pair);
    const int k = blockIdx.x;
    const int64_t n = b.n[k];
    O *out = static_cast<O *>(b.out[k]);
    for (int64_t i = n / kGroup * kGroup + threadIdx.x; i < n; i += kThreads)
        dequantize_one<O>(b.codes[k], i, b.absmax[k], b.q[k], b.sc[k], out, s_pair);
}

template <typename O>
struct DequantBatchLauncher {
    DequantBatch b;
    int count = 0;
    uint32_t wgs = 0;
    bool tail, dq;
    const Levels &lv;
    hipStream_t s;
    hipError_t err = hipSuccess;

    DequantBatchLauncher(bool tail_, bool dq_, const Levels &l, hipStream_t st)
        : tail(tail_), dq(dq_), lv(l), s(st) {}

    void flush() {
        if (count == 0) return;
        for (int j = count; j < kBatch; ++j) {
            b.codes[j] = nullptr;
            b.absmax[j] = nullptr;
            b.q[j] = nullptr;
            b.sc[j] = nullptr;
            b.out[j] = nullptr;
            b.n[j] = 0;
            b.first[j] = UINT32_MAX;
        }
        if (tail)
            dequantize_batch_tail_kernel<O><<<dim3((unsigned)count), dim3(kThreads), 0, s>>>(b, lv);
        else if (dq)
            dequantize_batch_kernel<O, true><<<dim3(wgs), dim3(kThreads), 0, s>>>(b, lv);
        else
            dequantize_batch_kernel<O, false><<<dim3(wgs), dim3(kThreads), 0, s>>>(b, lv);
        const hipError_t e = hipGetLastError();
        if (err == hipSuccess) err = e;
        count = 0;
        wgs = 0;
    }

    void add(const nf4_batch_entry &e, int64_t units) {
        constexpr int64_t kMaxWgs = (int64_t(1) << 31) / kThreads;  // below 2^31 threads
        if (count == kBatch || (!tail && (int64_t)wgs + units > kMaxWgs)) flush();
        b.codes[count] = e.codes;
        b.absmax[count] = dq ? nullptr : e.absmax;
        b.q[count] = dq ? e.absmax_q : nullptr;
        b.sc[count] = dq ? e.absmax_scale : nullptr;
        b.out[count] = e.w;
        b.n[count] = e.n;
        b.first[count] = tail ? 0u : wgs;
        wgs += tail ? 1u : (uint32_t)units;
        ++count;
    }
};

template <typename O>
hipError_t launch_dequantize_batched_t(const nf4_batch_entry *e, int32_t count, hipStream_t s) {
    Levels lv;
    for (int i = 0; i < 16; ++i) lv.q[i] = kLevels[i];
    hipError_t err = hipSuccess;
    for (int dq = 1; dq >= 0; --dq) {
        DequantBatchLauncher<O> full(false, dq != 0, lv, s), tail(true, dq != 0, lv, s);
        for (int32_t i = 0; i < count; ++i) {
            if ((e[i].absmax_q != nullptr) != (dq != 0) || e[i].n <= 0) continue;
            const int64_t groups = e[i].n / kGroup;
            if (groups > 0) full.add(e[i], groups * kGroupWgs);
            if (e[i].n % kGroup) tail.add(e[i], 1);
        }
        full.flush();
        tail.flush();
        if (err == hipSuccess) err = full.err != hipSuccess ? full.err : tail.err;
    }
    return err;
}

template <typename O>
hipError_t launch_t(const uint8_t *codes, int64_t n, const float *absmax, const uint8_t *absmax_q,
                    const float *absmax_scale, O *out, const float *levels, hipStream_t s) {
    Levels lv;
    for (int i = 0; i < 16; ++i) lv.q[i] = levels[i];
    constexpr int kCPW = 2;
    const int64_t nchunks = n / kChunk;
    if (nchunks > 0) {
        const int64_t waves = (nchunks + kCPW - 1) / kCPW;
        const int64_t wgs = (waves + (kThreads / 64) - 1) / (kThreads / 64);
        if (absmax_q)
            dequantize_chunks_kernel<O, true, kCPW><<<dim3((unsigned)wgs), dim3(kThreads), 0, s>>>(
                codes, nchunks, absmax, absmax_q, absmax_scale, out, lv);
        else
            dequantize_chunks_kernel<O, false, kCPW><<<dim3((unsigned)wgs), dim3(kThreads), 0, s>>>(
                codes, nchunks, absmax, absmax_q, absmax_scale, out, lv);
    }
    const int64_t start = nchunks * kChunk;
    if (start < n) {
        const int64_t rem = n - start;
        dequantize_tail_kernel<O><<<dim3((unsigned)((rem + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(
            codes, start, n, absmax, absmax_q, absmax_scale, out, lv);
    }
    return hipGetLastError();
}

// ---- storage-format variants: any block sizes, the 8-bit code format F
// and the mean offset (kS) ----

// Scale of block blk: absmax (kDQ false), or decode(q) * group value (+ mu).
template <int F, bool kS, bool kDQ>
struct VariantScale {
    const float *absmax;
    const uint8_t *q;
    const float *sc;
    float mu;
    int lb2;
    __device__ __forceinline__ float operator()(int64_t blk) const {
        if constexpr (!kDQ) {
            return absmax[blk];
        } else {
            float v = dq_decode<F, kS>((uint32_t)q[blk]) * sc[blk >> lb2];
            if constexpr (kS) v = v + mu;
            return v;
        }
    }
};

// The chunk kernel's layout (a wave owns 2048-weight chunks, lane l reads
// code dwords j * 256 + 4 l) with each lane's scale looked up per dword: the
// 8 weights of a dword lie in one block for every B1 >= 16.
template <typename O, int F, bool kS, bool kDQ, int kCPW>
__global__ __launch_bounds__(kThreads) void dequantize_variant_kernel(
    const uint8_t *__restrict__ codes, int64_t nchunks, int lb1, int lb2,
    const float *__restrict__ absmax, const uint8_t *__restrict__ absmax_q,
    const float *__restrict__ absmax_scale, const float *__restrict__ mu_p, O *__restrict__ out,
    Levels lv) {
    __shared__ float2 s_pair[256];
    __shared__ float s_lv[16];
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) +
                         __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    uint32_t d[kCPW][4];
#pragma unroll
    for (int c = 0; c < kCPW; ++c) {
        const int64_t chunk = min(wave * kCPW + c, nchunks - 1);
        const uint32_t *src = reinterpret_cast<const uint32_t *>(codes + chunk * kChunkBytes);
#pragma unroll
        for (int j = 0; j < 4; ++j) d[c][j] = __builtin_nontemporal_load(&src[j * 64 + lane]);
    }
    const VariantScale<F, kS, kDQ> scale{absmax, absmax_q, absmax_scale,
                                         (kDQ && kS) ? *mu_p : 0.0f, lb2};
    build_pair_table(lv, s_lv, s_pair);

#pragma unroll
    for (int c = 0; c < kCPW; ++c) {
        const int64_t chunk = wave * kCPW + c;
        if (chunk >= nchunks) return;
        float s[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = scale((chunk * kChunk + j * 512 + lane * 8) >> lb1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float2 qq = s_pair[(d[c][j] >> (8 * k)) & 0xFFu];
                v[2 * k] = qq.x * s[j];
                v[2 * k + 1] = qq.y * s[j];
            }
            Out<O>::store8(out + chunk * kChunk + j * 512 + lane * 8, v);
        }
    }
}

template <typename O, int F, bool kS, bool kDQ>
__global__ __launch_bounds__(kThreads) void dequantize_variant_tail_kernel(
    const uint8_t *__restrict__ codes, int64_t start, int64_t n, int lb1, int lb2,
    const float *__restrict__ absmax, const uint8_t *__restrict__ absmax_q,
    const float *__restrict__ absmax_scale, const float *__restrict__ mu_p, O *__restrict__ out,
    Levels lv) {
    __shared__ float2 s_pair[256];
    __shared__ float s_lv[16];
    build_pair_table(lv, s_lv, s_pair);
    const int64_t i = start + (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const VariantScale<F, kS, kDQ> scale{absmax, absmax_q, absmax_scale,
                                         (kDQ && kS) ? *mu_p : 0.0f, lb2};
    const uint32_t code = (codes[i >> 1] >> (4 * (i & 1))) & 15u;
    Out<O>::store1(out + i, s_pair[code].x * scale(i >> lb1));
}

template <typename O, int F, bool kS, bool kDQ>
hipError_t launch_variant(const uint8_t *codes, int64_t n, int lb1, int lb2, const float *absmax,
                          const uint8_t *q, const float *sc, const float *mu, O *out,
                          const float *levels, hipStream_t s) {
    Levels lv;
    for (int i = 0; i < 16; ++i) lv.q[i] = levels[i];
    constexpr int kCPW = 2;
    const int64_t nchunks = n / kChunk;
    if (nchunks > 0) {
        const int64_t waves = (nchunks + kCPW - 1) / kCPW;
        const int64_t wgs = (waves + (kThreads / 64) - 1) / (kThreads / 64);
        dequantize_variant_kernel<O, F, kS, kDQ, kCPW><<<dim3((unsigned)wgs), dim3(kThreads), 0, s>>>(
            codes, nchunks, lb1, lb2, absmax, q, sc, mu, out, lv);
    }
    const int64_t start = nchunks * kChunk;
    if (start < n) {
        const int64_t rem = n - start;
        dequantize_variant_tail_kernel<O, F, kS, kDQ>
            <<<dim3((unsigned)((rem + kThreads - 1) / kThreads)), dim3(kThreads), 0, s>>>(
                codes, start, n, lb1, lb2, absmax, q, sc, mu, out, lv);
    }
    return hipGetLastError();
}

template <typename O>
hipError_t launch_variant_o(const uint8_t *codes, int64_t n, const nf4_format &f,
                            const float *absmax, const uint8_t *q, const float *sc,
                            const float *mu, O *out, hipStream_t s) {
    const float *levels = levels_for(f.codebook);
    int lb1 = 0, lb2 = 0;
    while ((1 << lb1) < f.blocksize) ++lb1;
    while ((1 << lb2) < f.dq_blocksize) ++lb2;
    if (!q) return launch_variant<O, kFmtE4M3, false, false>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
    if (f.dq_mean_offset) {
        switch (f.dq_format) {
            case kFmtE5M2: return launch_variant<O, kFmtE5M2, true, true>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
            case kFmtLin8: return launch_variant<O, kFmtLin8, true, true>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
            default: return launch_variant<O, kFmtE4M3, true, true>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
        }
    }
    switch (f.dq_format) {
        case kFmtE5M2: return launch_variant<O, kFmtE5M2, false, true>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
        case kFmtLin8: return launch_variant<O, kFmtLin8, false, true>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
        default: return launch_variant<O, kFmtE4M3, false, true>(codes, n, lb1, lb2, absmax, q, sc, mu, out, levels, s);
    }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *codes, int64_t n, const float *absmax,
                             const uint8_t *absmax_q, const float *absmax_scale, void *out,
                             nf4_dtype dt, hipStream_t s) {
    if (dt == NF4_BF16)
        return launch_t<uint16_t>(codes, n, absmax, absmax_q, absmax_scale,
                                  static_cast<uint16_t *>(out), kLevels, s);
    return launch_t<float>(codes, n, absmax, absmax_q, absmax_scale, static_cast<float *>(out),
                           kLevels, s);
}

hipError_t launch_dequantize_batched(const nf4_batch_entry *e, int32_t count, nf4_dtype dt,
                                     hipStream_t s) {
    if (dt == NF4_BF16) return launch_dequantize_batched_t<uint16_t>(e, count, s);
    return launch_dequantize_batched_t<float>(e, count, s);
}

hipError_t launch_dequantize_ex(const uint8_t *codes, int64_t n, const nf4_format &f,
                                const float *absmax, const uint8_t *absmax_q,
                                const float *absmax_scale, const float *absmax_offset, void *out,
                                nf4_dtype dt, hipStream_t s) {
    const bool plain = f.blocksize == kBlock &&
                       (!absmax_q || (f.dq_blocksize == kDqBlock && f.dq_format == kFmtE4M3 &&
                                      !f.dq_mean_offset));
    if (plain) {
        const float *levels = levels_for(f.codebook);
        if (dt == NF4_BF16)
            return launch_t<uint16_t>(codes, n, absmax, absmax_q, absmax_scale,
                                      static_cast<uint16_t *>(out), levels, s);
        return launch_t<float>(codes, n, absmax, absmax_q, absmax_scale, static_cast<float *>(out),
                               levels, s);
    }
    if (dt == NF4_BF16)
        return launch_variant_o<uint16_t>(codes, n, f, absmax, absmax_q, absmax_scale,
                                          absmax_offset, static_cast<uint16_t *>(out), s);
    return launch_variant_o<float>(codes, n, f, absmax, absmax_q, absmax_scale, absmax_offset,
                                   static_cast<float *>(out), s);
}

}  // namespace nf4
