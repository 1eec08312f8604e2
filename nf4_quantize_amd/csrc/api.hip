// api.hip - the extern "C" entry points of libnf4.so: host-side validation,
// the NF4 code table, and dispatch to the gfx950 kernels. Declarations and
// the contract of each entry point are in include/nf4.h.
//
// Every argument is checked before any HIP call; a rejected call launches
// nothing and returns its status. The library allocates nothing.
#pragma clang fp contract(off)

#include <math.h>
#include <string.h>

#include <mutex>

#include "linear_common.h"

#define NF4_API extern "C" __attribute__((visibility("default")))

namespace nf4 {

// [MF] "4-Bit NormalFloat (NF4)": the printed list q_0 .. q_15 (each printed
// decimal is an exact binary32 value).
const float kLevels[16] = {
    -1.0f,
    -0.6961928009986877f,
    -0.5250730514526367f,
    -0.39491748809814453f,
    -0.28444138169288635f,
    -0.18477343022823334f,
    -0.09105003625154495f,
    0.0f,
    0.07958029955625534f,
    0.16093020141124725f,
    0.24611230194568634f,
    0.33791524171829224f,
    0.44070982933044434f,
    0.5626170039176941f,
    0.7229568362236023f,
    1.0f,
};

namespace {

// The other codebooks (nf4.h, nf4_codebook_id), each level rounded once to
// fp32: FP4 in the OCP E2M1 encoding (code = 8 * sign + magnitude index of
// {0, 0.5, 1, 1.5, 2, 3, 4, 6}) divided by 6, and evenly spaced Int4 levels.
struct OtherLevels {
    float fp4[16];
    float int4[16];
    OtherLevels() {
        const float e2m1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
        for (int i = 0; i < 8; ++i) {
            fp4[i] = e2m1[i] / 6.0f;
            fp4[8 + i] = -(e2m1[i] / 6.0f);
        }
        for (int k = 0; k < 16; ++k) int4[k] = (float)(2 * k - 15) / 15.0f;
    }
};
const OtherLevels &other_levels() {
    static const OtherLevels l;
    return l;
}

// Nearest level of a normalised value by direct search: the first index with
// the smallest |fl32(n - q_i)| ([MF] "Block-Wise Quantization Mechanics").
// Host-side only, used to build the bucket table.
int nearest_by_search(const float *lv, float n) {
    int best = 0;
    float bd = fabsf(n - lv[0]);
    for (int i = 1; i < 16; ++i) {
        const float d = fabsf(n - lv[i]);
        if (d < bd) {
            bd = d;
            best = i;
        }
    }
    return best;
}

// Total order of binary32 values as integers (for bisection over floats).
int64_t f2ord(float x) {
    uint32_t b;
    memcpy(&b, &x, 4);
    return (b & 0x80000000u) ? -(int64_t)(b & 0x7FFFFFFFu) : (int64_t)b;
}
float ord2f(int64_t o) {
    uint32_t b = o >= 0 ? (uint32_t)o : (0x80000000u | (uint32_t)(-o));
    float x;
    memcpy(&x, &b, 4);
    return x;
}

// Bucket of v, with the same fp32 formula as the kernels (see CodeLut).
uint32_t bucket_of(float v) { return lut_offset_bits(fmaf(v, 128.0f, 128.0f + 0x1p23f)) >> 3; }

// The code function the table encodes: the nearest level of v, or, for a
// sign-magnitude codebook (looked up with |v|), the nearest level of v >= 0
// and a constant 0 below zero (those buckets are never read).
int table_code(const float *lv, bool signmag, float v) {
    return (signmag && v < 0.0f) ? 0 : nearest_by_search(lv, v);
}

bool build_lut(CodeLut *lut, const float *lv, bool signmag) {
    const float vmin = -1.0f - 0x1p-20f, vmax = 1.0f + 0x1p-20f;
    auto code = [&](float v) { return table_code(lv, signmag, v); };
    // bucket_of is non-decreasing in v, so each bucket is an interval of floats.
    int64_t start = f2ord(vmin);
    const int64_t end = f2ord(vmax);
    if (bucket_of(vmin) != 0 || bucket_of(vmax) != kLutUsed - 1) return false;
    for (int k = 0; k < kLutUsed; ++k) {
        // last float of bucket k: bisection for the largest ordinal with bucket <= k
        int64_t a = start, b = end;
        if (bucket_of(ord2f(b)) <= (uint32_t)k) {
            a = b;
        } else {
            while (b - a > 1) {
                const int64_t mid = a + (b - a) / 2;
                if (bucket_of(ord2f(mid)) <= (uint32_t)k) a = mid; else b = mid;
            }
        }
        const float lo = ord2f(start), hi = ord2f(a);
        if (bucket_of(lo) != (uint32_t)k || bucket_of(hi) != (uint32_t)k) return false;
        const int c_lo = code(lo);
        const int c_hi = code(hi);
        lut->e[k].hi = c_hi;
        lut->e[k].thr = -2.0f;
        if (c_hi != c_lo) {
            if (c_hi != c_lo + 1) return false;  // more than one switch in a bucket
            int64_t u = f2ord(lo), v = f2ord(hi);  // code(u) == c_lo, code(v) == c_lo + 1
            while (v - u > 1) {
                const int64_t mid = u + (v - u) / 2;
                if (code(ord2f(mid)) > c_lo) v = mid; else u = mid;
            }
            const float thr = ord2f(v);
            // A switch point must sit inside its bucket by more than the
            // |q - n| bound (2.4e-7), so that q and n can only straddle the
            // switch point of the bucket q falls in (which the kernels test).
            if (!(thr - lo >= 0x1p-16f && hi - thr >= 0x1p-16f)) return false;
            lut->e[k].thr = thr;
        }
        start = a + 1;
    }
    for (int k = kLutUsed; k < kLutEntries; ++k) lut->e[k] = LutEntry{-2.0f, nearest_by_search(lv, 1.0f)};
    // the code of 0 (a block with c1 == 0) must come out of the table
    const LutEntry &z = lut->e[bucket_of(0.0f)];
    if (!(lut->e[kLutUsed - 1].hi == nearest_by_search(lv, 1.0f) &&
          z.hi - (0.0f < z.thr ? 1 : 0) == nearest_by_search(lv, 0.0f)))
        return false;
    if (signmag) {
        // code 8 + m is the mirror of magnitude code m, +0 is code 0 and -0
        // code 8, and every magnitude code in the table is below 8
        for (int m = 0; m < 8; ++m)
            if (!(lv[8 + m] == -lv[m])) return false;
        if (!(lv[0] == 0.0f && !signbit(lv[0]) && signbit(lv[8]))) return false;
        for (int k = 0; k < kLutEntries; ++k)
            if (lut->e[k].hi >= 8) return false;
    }
    return true;
}

}  // namespace

const float *levels_for(int cb) {
    switch (cb) {
        case NF4_CODEBOOK_NF4: return kLevels;
        case NF4_CODEBOOK_FP4: return other_levels().fp4;
        case NF4_CODEBOOK_INT4: return other_levels().int4;
        default: return nullptr;
    }
}

const CodeLut *code_lut_for(int cb) {
    static CodeLut lut[3];
    static bool ok[3] = {false, false, false};
    static std::once_flag once[3];
    if (cb < 0 || cb > 2) return nullptr;
    std::call_once(once[cb], [cb] {
        lut[cb].signmag = cb == NF4_CODEBOOK_FP4;
        ok[cb] = build_lut(&lut[cb], levels_for(cb), lut[cb].signmag != 0);
        lut[cb].refine = cb != NF4_CODEBOOK_NF4;
    });
    return ok[cb] ? &lut[cb] : nullptr;
}

const CodeLut *code_lut() { return code_lut_for(NF4_CODEBOOK_NF4); }

}  // namespace nf4

using namespace nf4;

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 37;  // keeps every grid below 2^32 threads

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

nf4_status launch_status(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_LAUNCH; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

NF4_API const char *nf4_status_string(int status) {
    switch (status) {
        case NF4_OK: return "NF4_OK";
        case NF4_ERR_NULL: return "NF4_ERR_NULL: a required pointer is NULL";
        case NF4_ERR_SIZE: return "NF4_ERR_SIZE: size out of range";
        case NF4_ERR_UNSUPPORTED: return "NF4_ERR_UNSUPPORTED: block size, dtype or format not supported";
        case NF4_ERR_ALIGN: return "NF4_ERR_ALIGN: buffer not aligned as required";
        case NF4_ERR_WORKSPACE: return "NF4_ERR_WORKSPACE: workspace missing or too small";
        case NF4_ERR_LAUNCH: return "NF4_ERR_LAUNCH: the HIP runtime reported a launch error";
        default: return "unknown nf4_status";
    }
}

NF4_API const float *nf4_codebook(void) { return kLevels; }

NF4_API const float *nf4_codebook_levels(int32_t codebook) { return levels_for(codebook); }

NF4_API int64_t nf4_storage_bytes(int64_t n, int32_t blocksize, int32_t dq_blocksize,
                                  int32_t double_quant) {
    if (n < 0 || blocksize != kBlock || (double_quant && dq_blocksize != kDqBlock)) return -1;
    const int64_t nb = cdiv(n, kBlock);
    const int64_t codes = cdiv(n, 2);
    if (!double_quant) return codes + 4 * nb;
    return codes + nb + 4 * cdiv(nb, kDqBlock);
}

NF4_API nf4_status nf4_quantize(const void *w, int32_t w_dtype, int64_t n, int32_t blocksize,
                                uint8_t *codes, float *absmax, int32_t dq_blocksize,
                                uint8_t *absmax_q, float *absmax_scale, void *stream) {
    if (n < 0 || n > kMaxElems) return NF4_ERR_SIZE;
    if (blocksize != kBlock) return NF4_ERR_UNSUPPORTED;
    if (w_dtype != NF4_F32 && w_dtype != NF4_BF16) return NF4_ERR_UNSUPPORTED;
    const bool dq = absmax_q != nullptr || absmax_scale != nullptr;
    if (dq && dq_blocksize != kDqBlock) return NF4_ERR_UNSUPPORTED;
    if (!code_lut()) return NF4_ERR_UNSUPPORTED;  // codebook table failed its checks
    if (n == 0) return NF4_OK;
    if (!w || !codes) return NF4_ERR_NULL;
    if (dq && (!absmax_q || !absmax_scale)) return NF4_ERR_NULL;
    if (!dq && !absmax) return NF4_ERR_NULL;
    if (!aligned(w, 16) || !aligned(codes, 16)) return NF4_ERR_ALIGN;
    if ((absmax && !aligned(absmax, 4)) || (absmax_q && !aligned(absmax_q, 4)) ||
        (absmax_scale && !aligned(absmax_scale, 4)))
        return NF4_ERR_ALIGN;
    return launch_status(launch_quantize(w, static_cast<nf4_dtype>(w_dtype), n, codes, absmax, absmax_q, absmax_scale,
                                         static_cast<hipStream_t>(stream)));
}

NF4_API nf4_status nf4_double_quantize(const float *absmax, int64_t nblocks, int32_t dq_blocksize,
                                       uint8_t *absmax_q, float *absmax_scale, void *stream) {
    if (nblocks < 0 || nblocks > kMaxElems / kBlock) return NF4_ERR_SIZE;
    if (dq_blocksize != kDqBlock) return NF4_ERR_UNSUPPORTED;
    if (nblocks == 0) return NF4_OK;
    if (!absmax || !absmax_q || !absmax_scale) return NF4_ERR_NULL;
    if (!aligned(absmax, 4) || !aligned(absmax_q, 4) || !aligned(absmax_scale, 4))
        return NF4_ERR_ALIGN;
    return launch_status(launch_double_quantize(absmax, nblocks, absmax_q, absmax_scale,
                                                static_cast<hipStream_t>(stream)));
}

NF4_API nf4_status nf4_dequantize(const uint8_t *codes, int64_t n, int32_t blocksize,
                                  const float *absmax, const uint8_t *absmax_q,
                                  const float *absmax_scale, int32_t dq_blocksize, void *out,
                                  int32_t out_dtype, void *stream) {
    if (n < 0 || n > kMaxElems) return NF4_ERR_SIZE;
    if (blocksize != kBlock) return NF4_ERR_UNSUPPORTED;
    if (out_dtype != NF4_F32 && out_dtype != NF4_BF16) return NF4_ERR_UNSUPPORTED;
    const bool dq = absmax_q != nullptr || absmax_scale != nullptr;
    if (dq && dq_blocksize != kDqBlock) return NF4_ERR_UNSUPPORTED;
    if (n == 0) return NF4_OK;
    if (!codes || !out) return NF4_ERR_NULL;
    if (dq && (!absmax_q || !absmax_scale)) return NF4_ERR_NULL;
    if (!dq && !absmax) return NF4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(out, 16)) return NF4_ERR_ALIGN;
    if ((absmax && !aligned(absmax, 4)) || (absmax_q && !aligned(absmax_q, 4)) ||
        (absmax_scale && !aligned(absmax_scale, 4)))
        return NF4_ERR_ALIGN;
    return launch_status(launch_dequantize(codes, n, dq ? nullptr : absmax, dq ? absmax_q : nullptr,
                                           dq ? absmax_scale : nullptr, out, static_cast<nf4_dtype>(out_dtype),
                                           static_cast<hipStream_t>(stream)));
}

namespace {

// One entry of a batched call: the checks of nf4_quantize / nf4_dequantize.
nf4_status check_batch_entry(const nf4_batch_entry &e) {
    if (e.n < 0 || e.n > kMaxElems) return NF4_ERR_SIZE;
    if (e.n == 0) return NF4_OK;
    const bool dq = e.absmax_q != nullptr || e.absmax_scale != nullptr;
    if (!e.w || !e.codes) return NF4_ERR_NULL;
    if (dq && (!e.absmax_q || !e.absmax_scale)) return NF4_ERR_NULL;
    if (!dq && !e.absmax) return NF4_ERR_NULL;
    if (!aligned(e.w, 16) || !aligned(e.codes, 16)) return NF4_ERR_ALIGN;
    if ((e.absmax && !aligned(e.absmax, 4)) || (e.absmax_q && !aligned(e.absmax_q, 4)) ||
        (e.absmax_scale && !aligned(e.absmax_scale, 4)))
        return NF4_ERR_ALIGN;
    return NF4_OK;
}

nf4_status check_batch(const nf4_batch_entry *entries, int32_t count, int32_t dt) {
    if (count < 0) return NF4_ERR_SIZE;
    if (dt != NF4_F32 && dt != NF4_BF16) return NF4_ERR_UNSUPPORTED;
    if (count > 0 && !entries) return NF4_ERR_NULL;
    for (int32_t i = 0; i < count; ++i) {
        const nf4_status st = check_batch_entry(entries[i]);
        if (st != NF4_OK) return st;
    }
    return NF4_OK;
}

}  // namespace

NF4_API nf4_status nf4_quantize_batched(const nf4_batch_entry *entries, int32_t count,
                                        int32_t w_dtype, void *stream) {
    const nf4_status st = check_batch(entries, count, w_dtype);
    if (st != NF4_OK) return st;
    if (!code_lut()) return NF4_ERR_UNSUPPORTED;  // codebook table failed its checks
    if (count == 0) return NF4_OK;
    return launch_status(
        launch_quantize_batched(entries, count, static_cast<nf4_dtype>(w_dtype), static_cast<hipStream_t>(stream)));
}

NF4_API nf4_status nf4_dequantize_batched(const nf4_batch_entry *entries, int32_t count,
                                          int32_t out_dtype, void *stream) {
    const nf4_status st = check_batch(entries, count, out_dtype);
    if (st != NF4_OK) return st;
    if (count == 0) return NF4_OK;
    return launch_status(
        launch_dequantize_batched(entries, count, static_cast<nf4_dtype>(out_dtype), static_cast<hipStream_t>(stream)));
}

NF4_API size_t nf4_linear_workspace_size(int64_t m, int32_t r) {
    if (m <= 0 || r <= 0) return 0;
    return nf4::lora_workspace_bytes(m, ((int64_t)r + 63) / 64 * 64);
}

namespace {

// Everything of a linear call but its workspace.
nf4_status check_linear_args(const void *act, int64_t m, const nf4_weight *w, const void *a,
                             const void *b, int32_t r, const void *out) {
    if (!w) return NF4_ERR_NULL;
    if (m < 0 || w->n_out <= 0 || w->k_in <= 0 || (w->k_in % kBlock) != 0) return NF4_ERR_SIZE;
    if (w->n_out * w->k_in > kMaxElems || m > (int64_t(1) << 31)) return NF4_ERR_SIZE;
    if (m * w->k_in > kMaxElems || m * w->n_out > kMaxElems) return NF4_ERR_SIZE;
    if (r < 0 || r > 256) return NF4_ERR_SIZE;
    if (w->blocksize != kBlock) return NF4_ERR_UNSUPPORTED;
    const bool dq = w->absmax_q != nullptr || w->absmax_scale != nullptr;
    if (dq && w->dq_blocksize != kDqBlock) return NF4_ERR_UNSUPPORTED;
    if (m == 0) return NF4_OK;
    if (!act || !out || !w->codes) return NF4_ERR_NULL;
    if (dq && (!w->absmax_q || !w->absmax_scale)) return NF4_ERR_NULL;
    if (!dq && !w->absmax) return NF4_ERR_NULL;
    if ((r > 0) != (a != nullptr) || (r > 0 && !b)) return NF4_ERR_NULL;
    if (!aligned(act, 16) || !aligned(out, 16) || !aligned(w->codes, 16)) return NF4_ERR_ALIGN;
    if ((w->absmax && !aligned(w->absmax, 4)) || (w->absmax_q && !aligned(w->absmax_q, 4)) ||
        (w->absmax_scale && !aligned(w->absmax_scale, 4)))
        return NF4_ERR_ALIGN;
    if (r > 0 && (!aligned(a, 16) || !aligned(b, 16))) return NF4_ERR_ALIGN;
    return NF4_OK;
}

nf4_status check_linear(const void *act, int64_t m, const nf4_weight *w, const void *a,
                        const void *b, int32_t r, const void *out, const void *ws,
                        size_t ws_bytes) {
    const nf4_status st = check_linear_args(act, m, w, a, b, r, out);
    if (st != NF4_OK || m == 0) return st;
    if (r > 0) {
        if (!ws || ws_bytes < nf4_linear_workspace_size(m, r)) return NF4_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return NF4_ERR_ALIGN;
    }
    return NF4_OK;
}

nf4_weight normalised(const nf4_weight *w) {
    nf4_weight v = *w;
    if (v.absmax_q) v.absmax = nullptr;
    return v;
}

}  // namespace

NF4_API nf4_status nf4_linear_forward(const void *x, int64_t m, const nf4_weight *w,
                                      const void *lora_a, const void *lora_b, int32_t r,
                                      float lora_scale, void *y, void *workspace,
                                      size_t workspace_bytes, void *stream) {
    const nf4_status st = check_linear(x, m, w, lora_a, lora_b, r, y, workspace, workspace_bytes);
    if (st != NF4_OK || m == 0) return st;
    return launch_status(launch_linear_forward(
        static_cast<const uint16_t *>(x), m, normalised(w), static_cast<const uint16_t *>(lora_a),
        static_cast<const uint16_t *>(lora_b), r, lora_scale, static_cast<uint16_t *>(y),
        workspace, static_cast<hipStream_t>(stream)));
}

namespace {

// The scratch of nf4_linear_forward_noalloc: the adapter product and its
// split-K partial sums, the same bytes nf4_linear_forward takes as its
// workspace, in a device array that every call on a GPU shares. In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device, with
// that device current, and only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[NF4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void *ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot &slot = g_scratch[dev];
    std::call_once(slot.once, [&slot] {
        slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess && !slot.ptr) slot.err = hipErrorInvalidSymbol;
    });
    if (slot.err != hipSuccess) return slot.err;
    *out = slot.ptr;
    return hipSuccess;
}

}  // namespace

NF4_API nf4_status nf4_linear_forward_noalloc(const void *x, int64_t m, const nf4_weight *w,
                                              const void *lora_a, const void *lora_b, int32_t r,
                                              float lora_scale, void *y, void *stream) {
    const nf4_status st = check_linear_args(x, m, w, lora_a, lora_b, r, y);
    if (st != NF4_OK || m == 0) return st;
    const size_t need = nf4_linear_workspace_size(m, r);
    if (need > (size_t)NF4_NOALLOC_SCRATCH_BYTES) return NF4_ERR_SIZE;
    void *ws = nullptr;
    if (need > 0 && scratch_address(&ws) != hipSuccess) return NF4_ERR_LAUNCH;
    return launch_status(launch_linear_forward(
        static_cast<const uint16_t *>(x), m, normalised(w), static_cast<const uint16_t *>(lora_a),
        static_cast<const uint16_t *>(lora_b), r, lora_scale, static_cast<uint16_t *>(y), ws,
        static_cast<hipStream_t>(stream)));
}

NF4_API nf4_status nf4_linear_backward_input(const void *dy, int64_t m, const nf4_weight *w,
                                             const void *lora_a, const void *lora_b, int32_t r,
                                             float lora_scale, void *dx, void *workspace,
                                             size_t workspace_bytes, void *stream) {
    const nf4_status st = check_linear(dy, m, w, lora_a, lora_b, r, dx, workspace, workspace_bytes);
    if (st != NF4_OK || m == 0) return st;
    return launch_status(launch_linear_backward_input(
        static_cast<const uint16_t *>(dy), m, normalised(w), static_cast<const uint16_t *>(lora_a),
        static_cast<const uint16_t *>(lora_b), r, lora_scale, static_cast<uint16_t *>(dx),
        workspace, static_cast<hipStream_t>(stream)));
}

NF4_API int32_t nf4_linear_kernel_path(int64_t m, int64_t n_out, int64_t k_in, int32_t r, int32_t backward) {
    if (m < 0 || n_out < 1 || k_in < 1 || k_in % kBlock != 0 || r < 0 || r > 256) return -1;
    return (int32_t)linear_path(m, n_out, k_in, r, backward != 0);
}

NF4_API size_t nf4_lora_backward_workspace_size(int64_t m, int64_t k_in, int64_t n_out, int32_t r) {
    if (m < 0 || k_in <= 0 || n_out <= 0 || r <= 0 || r > 256) return 0;
    return nf4::lora_grads_workspace_bytes(m, k_in, n_out, ((int64_t)r + 63) / 64 * 64, r);
}

NF4_API nf4_status nf4_lora_backward(const void *x, const void *dy, int64_t m, int64_t k_in, int64_t n_out,
                                     const void *lora_a, const void *lora_b, int32_t r, float lora_scale,
                                     void *grad_a, void *grad_b, int32_t grad_dtype, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (m < 0 || k_in <= 0 || n_out <= 0 || (k_in % 64) != 0 || (n_out % 64) != 0) return NF4_ERR_SIZE;
    if (r <= 0 || r > 256 || (r % 8) != 0) return NF4_ERR_SIZE;
    if (m > (int64_t(1) << 31) || m * k_in > kMaxElems || m * n_out > kMaxElems) return NF4_ERR_SIZE;
    if (k_in * r > kMaxElems || n_out * r > kMaxElems) return NF4_ERR_SIZE;
    if (grad_dtype != NF4_F32 && grad_dtype != NF4_BF16) return NF4_ERR_UNSUPPORTED;
    if (!grad_a && !grad_b) return NF4_OK;
    if (!lora_a || !lora_b || (m > 0 && (!x || !dy))) return NF4_ERR_NULL;
    if ((x && !aligned(x, 16)) || (dy && !aligned(dy, 16)) || !aligned(lora_a, 16) || !aligned(lora_b, 16) ||
        (grad_a && !aligned(grad_a, 16)) || (grad_b && !aligned(grad_b, 16)))
        return NF4_ERR_ALIGN;
    if (!workspace || workspace_bytes < nf4_lora_backward_workspace_size(m, k_in, n_out, r))
        return NF4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return NF4_ERR_ALIGN;
    return launch_status(nf4::launch_lora_grads(
        static_cast<const uint16_t *>(x), static_cast<const uint16_t *>(dy), m, k_in, n_out,
        static_cast<const uint16_t *>(lora_a), static_cast<const uint16_t *>(lora_b), r, lora_scale, grad_a,
        grad_b, grad_dtype == NF4_F32, workspace, static_cast<hipStream_t>(stream)));
}

// ---- storage-format variants ----

namespace {

bool pow2_in(int64_t v, int64_t lo, int64_t hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

nf4_status check_format(const nf4_format *f) {
    if (!f) return NF4_ERR_NULL;
    if (!pow2_in(f->blocksize, 16, 4096) || !pow2_in(f->dq_blocksize, 1, 4096))
        return NF4_ERR_UNSUPPORTED;
    if (f->dq_format < NF4_DQ_E4M3 || f->dq_format > NF4_DQ_LINEAR8) return NF4_ERR_UNSUPPORTED;
    if (f->dq_mean_offset != 0 && f->dq_mean_offset != 1) return NF4_ERR_UNSUPPORTED;
    if (!code_lut_for(f->codebook)) return NF4_ERR_UNSUPPORTED;
    return NF4_OK;
}

nf4_status check_workspace(size_t need, const void *ws, size_t ws_bytes) {
    if (need == 0) return NF4_OK;
    if (!ws || ws_bytes < need) return NF4_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return NF4_ERR_ALIGN;
    return NF4_OK;
}

}  // namespace

NF4_API int64_t nf4_storage_bytes_ex(int64_t n, const nf4_format *f, int32_t double_quant) {
    if (check_format(f) != NF4_OK || n < 0) return -1;
    const int64_t nb = cdiv(n, f->blocksize);
    const int64_t codes = cdiv(n, 2);
    if (!double_quant) return codes + 4 * nb;
    return codes + nb + 4 * cdiv(nb, f->dq_blocksize) + (f->dq_mean_offset ? 4 : 0);
}

NF4_API size_t nf4_quantize_ex_workspace_size(int64_t n, const nf4_format *f) {
    if (check_format(f) != NF4_OK || n < 0 || n > kMaxElems) return (size_t)-1;
    return nf4::quantize_ex_workspace(n, *f);
}

NF4_API size_t nf4_double_quantize_ex_workspace_size(int64_t nblocks, const nf4_format *f) {
    if (check_format(f) != NF4_OK || nblocks < 0 || nblocks > kMaxElems / 16) return (size_t)-1;
    return nf4::double_quantize_ex_workspace(nblocks, *f);
}

NF4_API nf4_status nf4_quantize_ex(const void *w, int32_t w_dtype, int64_t n, const nf4_format *f,
                                   uint8_t *codes, float *absmax, uint8_t *absmax_q,
                                   float *absmax_scale, float *absmax_offset, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    nf4_status st = check_format(f);
    if (st != NF4_OK) return st;
    if (n < 0 || n > kMaxElems) return NF4_ERR_SIZE;
    if (w_dtype != NF4_F32 && w_dtype != NF4_BF16) return NF4_ERR_UNSUPPORTED;
    if (!code_lut()) return NF4_ERR_UNSUPPORTED;
    const bool dq = absmax_q != nullptr || absmax_scale != nullptr;
    if (n == 0) return NF4_OK;
    if (!w || !codes) return NF4_ERR_NULL;
    if (dq && (!absmax_q || !absmax_scale)) return NF4_ERR_NULL;
    if (!dq && !absmax) return NF4_ERR_NULL;
    if (dq && f->dq_mean_offset && !absmax_offset) return NF4_ERR_NULL;
    if (!aligned(w, 16) || !aligned(codes, 16)) return NF4_ERR_ALIGN;
    if ((absmax && !aligned(absmax, 4)) || (absmax_q && !aligned(absmax_q, 4)) ||
        (absmax_scale && !aligned(absmax_scale, 4)) || (absmax_offset && !aligned(absmax_offset, 4)))
        return NF4_ERR_ALIGN;
    if (dq && (st = check_workspace(nf4::quantize_ex_workspace(n, *f), workspace,
                                    workspace_bytes)) != NF4_OK)
        return st;
    return launch_status(nf4::launch_quantize_ex(w, static_cast<nf4_dtype>(w_dtype), n, *f, codes, absmax,
                                                 dq ? absmax_q : nullptr,
                                                 dq ? absmax_scale : nullptr, absmax_offset,
                                                 workspace, static_cast<hipStream_t>(stream)));
}

NF4_API nf4_status nf4_double_quantize_ex(const float *absmax, int64_t nblocks, const nf4_format *f,
                                          uint8_t *absmax_q, float *absmax_scale,
                                          float *absmax_offset, void *workspace,
                                          size_t workspace_bytes, void *stream) {
    nf4_status st = check_format(f);
    if (st != NF4_OK) return st;
    if (nblocks < 0 || nblocks > kMaxElems / 16) return NF4_ERR_SIZE;
    if (nblocks == 0) return NF4_OK;
    if (!absmax || !absmax_q || !absmax_scale) return NF4_ERR_NULL;
    if (f->dq_mean_offset && !absmax_offset) return NF4_ERR_NULL;
    if (!aligned(absmax, 4) || !aligned(absmax_q, 4) || !aligned(absmax_scale, 4) ||
        (absmax_offset && !aligned(absmax_offset, 4)))
        return NF4_ERR_ALIGN;
    if ((st = check_workspace(nf4::double_quantize_ex_workspace(nblocks, *f), workspace,
                              workspace_bytes)) != NF4_OK)
        return st;
    return launch_status(nf4::launch_double_quantize_ex(absmax, nblocks, *f, absmax_q,
                                                        absmax_scale, absmax_offset, workspace,
                                                        static_cast<hipStream_t>(stream)));
}

NF4_API nf4_status nf4_dequantize_ex(const uint8_t *codes, int64_t n, const nf4_format *f,
                                     const float *absmax, const uint8_t *absmax_q,
                                     const float *absmax_scale, const float *absmax_offset,
                                     void *out, int32_t out_dtype, void *stream) {
    nf4_status st = check_format(f);
    if (st != NF4_OK) return st;
    if (n < 0 || n > kMaxElems) return NF4_ERR_SIZE;
    if (out_dtype != NF4_F32 && out_dtype != NF4_BF16) return NF4_ERR_UNSUPPORTED;
    const bool dq = absmax_q != nullptr || absmax_scale != nullptr;
    if (n == 0) return NF4_OK;
    if (!codes || !out) return NF4_ERR_NULL;
    if (dq && (!absmax_q || !absmax_scale)) return NF4_ERR_NULL;
    if (!dq && !absmax) return NF4_ERR_NULL;
    if (dq && f->dq_mean_offset && !absmax_offset) return NF4_ERR_NULL;
    if (!aligned(codes, 16) || !aligned(out, 16)) return NF4_ERR_ALIGN;
    if ((absmax && !aligned(absmax, 4)) || (absmax_q && !aligned(absmax_q, 4)) ||
        (absmax_scale && !aligned(absmax_scale, 4)) || (absmax_offset && !aligned(absmax_offset, 4)))
        return NF4_ERR_ALIGN;
    return launch_status(nf4::launch_dequantize_ex(
        codes, n, *f, dq ? nullptr : absmax, dq ? absmax_q : nullptr, dq ? absmax_scale : nullptr,
        (dq && f->dq_mean_offset) ? absmax_offset : nullptr, out, static_cast<nf4_dtype>(out_dtype),
        static_cast<hipStream_t>(stream)));
}

// ---- merging the adapter into the quantized base ----

NF4_API size_t nf4_merge_lora_workspace_size(int64_t n_out, int64_t k_in) {
    if (n_out <= 0 || k_in <= 0 || (k_in % kBlock) != 0 || n_out * k_in > kMaxElems) return 0;
    return nf4::merge_workspace(n_out, k_in);
}

NF4_API nf4_status nf4_merge_lora(const nf4_weight *w, const void *lora_a, const void *lora_b,
                                  int32_t r, float lora_scale, uint8_t *codes_out, float *absmax_out,
                                  uint8_t *absmax_q_out, float *absmax_scale_out, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    if (!w) return NF4_ERR_NULL;
    if (w->n_out <= 0 || w->k_in <= 0 || (w->k_in % kBlock) != 0) return NF4_ERR_SIZE;
    if (w->n_out * w->k_in > kMaxElems) return NF4_ERR_SIZE;
    if (r < 8 || r > 256 || (r % 8) != 0) return NF4_ERR_SIZE;
    if (w->blocksize != kBlock) return NF4_ERR_UNSUPPORTED;
    if (!code_lut()) return NF4_ERR_UNSUPPORTED;
    const bool dq_in = w->absmax_q != nullptr || w->absmax_scale != nullptr;
    if (dq_in && w->dq_blocksize != kDqBlock) return NF4_ERR_UNSUPPORTED;
    if (!w->codes || !lora_a || !lora_b || !codes_out) return NF4_ERR_NULL;
    if (dq_in && (!w->absmax_q || !w->absmax_scale)) return NF4_ERR_NULL;
    if (!dq_in && !w->absmax) return NF4_ERR_NULL;
    const bool dq_out = absmax_q_out != nullptr || absmax_scale_out != nullptr;
    if (dq_out && (!absmax_q_out || !absmax_scale_out)) return NF4_ERR_NULL;
    if (!dq_out && !absmax_out) return NF4_ERR_NULL;
    if (!aligned(w->codes, 16) || !aligned(codes_out, 16) || !aligned(lora_a, 16) ||
        !aligned(lora_b, 2))
        return NF4_ERR_ALIGN;
    if ((w->absmax && !aligned(w->absmax, 4)) || (w->absmax_q && !aligned(w->absmax_q, 4)) ||
        (w->absmax_scale && !aligned(w->absmax_scale, 4)) || (absmax_out && !aligned(absmax_out, 4)) ||
        (absmax_q_out && !aligned(absmax_q_out, 4)) ||
        (absmax_scale_out && !aligned(absmax_scale_out, 4)))
        return NF4_ERR_ALIGN;
    if (dq_out && !absmax_out) {
        const size_t need = nf4::merge_workspace(w->n_out, w->k_in);
        if (!workspace || workspace_bytes < need) return NF4_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return NF4_ERR_ALIGN;
    }
    nf4_weight wv = *w;
    if (!dq_in) wv.absmax_q = nullptr, wv.absmax_scale = nullptr;
    return launch_status(nf4::launch_merge(
        wv, static_cast<const uint16_t *>(lora_a), static_cast<const uint16_t *>(lora_b), r,
        lora_scale, codes_out, absmax_out, absmax_q_out, absmax_scale_out, workspace,
        static_cast<hipStream_t>(stream)));
}
