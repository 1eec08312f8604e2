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

}  // namespace

// kind 0: stream_r4w1, src >= groups * 32 KiB, dst >= groups * 8 KiB.
// kind 1: stream_r1w4, src >= groups * 8 KiB, dst >= groups * 32 KiB.
// kind 2: stream_r1w0, src >= groups * 32 KiB, dst >= groups * 16 B (key
//         0xFFFFFFFF: the caller fills src so that no thread's XOR has all bits set).
// Device buffers, 16-byte aligned; 0 < groups < 2^22. Returns a hipError_t.
extern "C" __attribute__((visibility("default"))) int bench_stream(int kind, const void *src,
                                                                   void *dst, int64_t groups,
                                                                   void *stream) {
    if (groups <= 0 || groups >= (int64_t(1) << 22) || !src || !dst ||
        (reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15))
        return (int)hipErrorInvalidValue;
    const hipStream_t s = static_cast<hipStream_t>(stream);
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
