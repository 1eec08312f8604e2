// bench_stream.hip - plain HBM streaming kernels for bench.py: the memory
// traffic of the storage path's two kernels with none of their arithmetic,
// so their measured time is the practical ceiling the quantize and
// dequantize kernels are compared with (next to the 8 TB/s published peak).
// Not part of libnf4.so; built into bench_stream.so.
//
// Both kernels work on "groups" of 16384 bf16 weights, one workgroup per group:
//   stream_r4w1 (quantize's traffic): reads 32 KiB, writes 8 KiB per group.
//     512 threads; thread t reads four 16-byte vectors at t, t+512, t+1024,
//     t+1536 (each wave instruction one contiguous 1 KiB run, issued together
//     as non-temporal loads) and writes their XOR as one 16-byte vector.
//   stream_r1w4 (dequantize's traffic): reads 8 KiB, writes 32 KiB per group.
//     256 threads; thread t reads two 16-byte vectors (t, t+256) and writes
//     four 16-byte vectors per read (v, v^1, v^2, v^3), every wave
//     instruction one contiguous 1 KiB run, stores non-temporal.
//   stream_r1w0 (the decode GEMV's weight stream): reads 32 KiB per group as
//     stream_r4w1 does and writes nothing unless the XOR of a thread's four
//     vectors equals `key` (the caller passes a key the data never forms, so
//     the loads stay and no store happens).
// Best-effort forms of the same three traffic patterns, free of the
// one-workgroup-per-group grid: stream_persistent<R, W> runs a grid of the
// caller's size (a few workgroups per CU) whose 256-thread workgroups walk
// the groups with a grid stride. Each thread handles R 16-byte reads and W
// 16-byte writes per group, and the loads of its next group are issued
// before the stores of the current one, so every thread keeps two groups'
// loads in flight. The caller sweeps the grid size and keeps the fastest.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

__global__ __launch_bounds__(512) void stream_r4w1(const u32x4 *__restrict__ src,
                                                   u32x4 *__restrict__ dst) {
    const int t = threadIdx.x;
    const u32x4 *s = src + (int64_t)blockIdx.x * 2048;
    const u32x4 a = __builtin_nontemporal_load(s + t);
    const u32x4 b = __builtin_nontemporal_load(s + 512 + t);
    const u32x4 c = __builtin_nontemporal_load(s + 1024 + t);
    const u32x4 d = __builtin_nontemporal_load(s + 1536 + t);
    __builtin_nontemporal_store(a ^ b ^ c ^ d, dst + (int64_t)blockIdx.x * 512 + t);
}

__global__ __launch_bounds__(256) void stream_r1w4(const u32x4 *__restrict__ src,
                                                   u32x4 *__restrict__ dst) {
    const int t = threadIdx.x;
    const u32x4 *s = src + (int64_t)blockIdx.x * 512;
    u32x4 *o = dst + (int64_t)blockIdx.x * 2048;
    const u32x4 v[2] = {__builtin_nontemporal_load(s + t), __builtin_nontemporal_load(s + 256 + t)};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 x = v[h] ^ (uint32_t)j;
            __builtin_nontemporal_store(x, o + h * 1024 + j * 256 + t);
        }
    }
}

__global__ __launch_bounds__(512) void stream_r1w0(const u32x4 *__restrict__ src,
                                                   u32x4 *__restrict__ dst, uint32_t key) {
    const int t = threadIdx.x;
    const u32x4 *s = src + (int64_t)blockIdx.x * 2048;
    const u32x4 a = __builtin_nontemporal_load(s + t);
    const u32x4 b = __builtin_nontemporal_load(s + 512 + t);
    const u32x4 c = __builtin_nontemporal_load(s + 1024 + t);
    const u32x4 d = __builtin_nontemporal_load(s + 1536 + t);
    const u32x4 x = a ^ b ^ c ^ d;
    if ((x.x | x.y | x.z | x.w) == key) dst[blockIdx.x] = x;
}

// R reads and W writes of 16 bytes per thread and group (256 threads): a
// group is 256 * R read vectors and 256 * W written vectors, each wave
// instruction one contiguous 1 KiB run. W == 0: the loads are kept by a
// store that never happens (key as in stream_r1w0).
template <int R, int W>
__global__ __launch_bounds__(256) void stream_persistent(const u32x4 *__restrict__ src,
                                                         u32x4 *__restrict__ dst, int64_t groups,
                                                         uint32_t key) {
    const int t = threadIdx.x;
    int64_t g = blockIdx.x;
    if (g >= groups) return;
    u32x4 v[R];
#pragma unroll
    for (int i = 0; i < R; ++i) v[i] = __builtin_nontemporal_load(src + g * (256 * R) + i * 256 + t);
    for (; g < groups; g += gridDim.x) {
        const int64_t gn = g + gridDim.x;
        u32x4 nv[R];
        if (gn < groups) {
#pragma unroll
            for (int i = 0; i < R; ++i)
                nv[i] = __builtin_nontemporal_load(src + gn * (256 * R) + i * 256 + t);
        }
        u32x4 x = v[0];
#pragma unroll
        for (int i = 1; i < R; ++i) x ^= v[i];
        if constexpr (W == 0) {
            if ((x.x | x.y | x.z | x.w) == key) dst[g] = x;
        } else {
#pragma unroll
            for (int j = 0; j < W; ++j)
                __builtin_nontemporal_store(x ^ (uint32_t)j, dst + g * (256 * W) + j * 256 + t);
        }
        if (gn < groups) {
#pragma unroll
            for (int i = 0; i < R; ++i) v[i] = nv[i];
        }
    }
}

// The matrix cores' practical ceiling on data (the bf16 MFMA of the fused
// GEMM, v_mfma_f32_32x32x16_bf16): each wave loads 8 A and 8 B operands
// (16 bytes per lane each, bf16 values from src) and issues 64 MFMAs per
// iteration, every one on a different (A, B) pair, into 4 accumulator tiles,
// so the operand bits change with every instruction as they do in a GEMM on
// real data (the matrix cores' power, and so the clock they hold, depends on
// it). No other instruction sits between the MFMAs. Each workgroup (4
// waves) writes its 4 waves' accumulators, 64 x 64 floats per wave.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__global__ __launch_bounds__(256) void mfma_ceiling(const u32x4 *__restrict__ src, int iters,
                                                    float *__restrict__ dst) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const u32x4 *s = src + (int64_t)(blockIdx.x * 4 + wv) * 16 * 64;
    u32x4 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = s[i * 64 + lane];
        b[i] = s[(8 + i) * 64 + lane];
    }
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int m = 0; m < 64; ++m)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                         : "+a"(acc[m % 4]) : "v"(a[m % 8]), "v"(b[(m / 8 + m) % 8]));
    }
    // wait states before the accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7");
    float *o = dst + (int64_t)(blockIdx.x * 4 + wv) * 4096;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[(t * 16 + v) * 64 + lane] = acc[t][v];
}

}  // namespace

// Runs mfma_ceiling on `grid` workgroups: src >= grid * 4 * 16 KiB of bf16,
// dst >= grid * 4 * 4096 floats, 16-byte aligned; 1 <= grid <= 65536,
// 1 <= iters <= 2^20. Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int bench_mfma(const void *src, void *dst, int grid,
                                                                 int iters, void *stream) {
    if (!src || !dst || grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 20) ||
        (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return (int)hipErrorInvalidValue;
    mfma_ceiling<<<dim3((unsigned)grid), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const u32x4 *>(src), iters, static_cast<float *>(dst));
    return (int)hipGetLastError();
}

// kind 0: stream_r4w1, src >= groups * 32 KiB, dst >= groups * 8 KiB.
// kind 1: stream_r1w4, src >= groups * 8 KiB, dst >= groups * 32 KiB.
// kind 2: stream_r1w0, src >= groups * 32 KiB, dst >= groups * 16 B (key
//         0xFFFFFFFF: the caller fills src so that no thread's XOR has all bits set).
// kind 3, 4, 5: the traffic of kinds 0, 1, 2 by stream_persistent on a grid
//         of `grid` workgroups (1 <= grid <= 65536; kinds 0..2 ignore it).
// Device buffers, 16-byte aligned; 0 < groups < 2^22. Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int bench_stream_grid(int kind, const void *src,
                                                                        void *dst, int64_t groups,
                                                                        int grid, void *stream) {
    if (groups <= 0 || groups >= (int64_t(1) << 22) || !src || !dst ||
        (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return (int)hipErrorInvalidValue;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (kind >= 3 && kind <= 5) {
        if (grid < 1 || grid > 65536) return (int)hipErrorInvalidValue;
        const u32x4 *a = static_cast<const u32x4 *>(src);
        u32x4 *b = static_cast<u32x4 *>(dst);
        if (kind == 3)
            stream_persistent<8, 2><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a, b, groups, 0u);
        else if (kind == 4)
            stream_persistent<2, 8><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a, b, groups, 0u);
        else
            stream_persistent<8, 0><<<dim3((unsigned)grid), dim3(256), 0, s>>>(a, b, groups,
                                                                               0xFFFFFFFFu);
        return (int)hipGetLastError();
    }
    if (kind == 0)
        stream_r4w1<<<dim3((unsigned)groups), dim3(512), 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst));
    else if (kind == 1)
        stream_r1w4<<<dim3((unsigned)groups), dim3(256), 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst));
    else if (kind == 2)
        stream_r1w0<<<dim3((unsigned)groups), dim3(512), 0, s>>>(
            static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), 0xFFFFFFFFu);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

extern "C" __attribute__((visibility("default"))) int bench_stream(int kind, const void *src,
                                                                   void *dst, int64_t groups,
                                                                   void *stream) {
    return kind <= 2 ? bench_stream_grid(kind, src, dst, groups, 1, stream)
                     : (int)hipErrorInvalidValue;
}
