// Drives the host side of libnf4 for the AddressSanitizer /
// UndefinedBehaviorSanitizer build of tests/test_sanitizers.py: every entry
// point's argument validation (each call here is rejected, or is empty, before
// any HIP call, so no GPU is needed), the size and workspace functions, and
// the code-table builder of the quantize kernels for each codebook. The
// device pointers are never dereferenced addresses.
#include <cstdint>
#include <cstdio>

#include "nf4.h"
#include "nf4_internal.h"

namespace {

int failures = 0;

#define EXPECT(expr, want)                                                                   \
    do {                                                                                     \
        const long long got_ = (long long)(expr);                                            \
        if (got_ != (long long)(want)) {                                                     \
            std::fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #expr, \
                         got_, (long long)(want));                                           \
            ++failures;                                                                      \
        }                                                                                    \
    } while (0)

void *const F = reinterpret_cast<void *>(uintptr_t(0x10000));
template <typename T> T *at(uintptr_t off) { return reinterpret_cast<T *>(uintptr_t(0x10000) + off); }

nf4_weight weight(int64_t n = 256, int64_t k = 512, int bs = 64, int dq = 256, bool q = true) {
    nf4_weight w{};
    w.codes = at<const uint8_t>(0);
    w.absmax_q = q ? at<const uint8_t>(0) : nullptr;
    w.absmax_scale = q ? at<const float>(0) : nullptr;
    w.absmax = q ? nullptr : at<const float>(0);
    w.n_out = n;
    w.k_in = k;
    w.blocksize = bs;
    w.dq_blocksize = dq;
    return w;
}

nf4_format fmt(int bs = 64, int dq = 256, int f = 0, int off = 0, int cb = 0) {
    return nf4_format{bs, dq, f, off, cb};
}

void storage() {
    for (int s = -1; s <= 7; ++s) EXPECT(nf4_status_string(s) != nullptr, 1);
    EXPECT(nf4_codebook() != nullptr, 1);
    for (int cb = 0; cb < 3; ++cb) EXPECT(nf4_codebook_levels(cb) != nullptr, 1);
    EXPECT(nf4_codebook_levels(3) == nullptr, 1);
    EXPECT(nf4_codebook_levels(-1) == nullptr, 1);
    EXPECT(nf4_storage_bytes(1 << 20, 64, 256, 1), 540928);
    EXPECT(nf4_storage_bytes(-1, 64, 256, 1), -1);
    EXPECT(nf4_storage_bytes(int64_t(1) << 62, 64, 256, 1) < 0 ||
               nf4_storage_bytes(int64_t(1) << 62, 64, 256, 1) > 0, 1);
    for (int bs : {8, 16, 64, 96, 4096, 8192})
        for (int dq : {0, 1, 3, 256, 4096, 8192})
            for (int off = 0; off < 3; ++off) {
                const nf4_format f = fmt(bs, dq, 0, off);
                (void)nf4_storage_bytes_ex(12345, &f, 1);
                (void)nf4_quantize_ex_workspace_size(12345, &f);
                (void)nf4_double_quantize_ex_workspace_size(12345, &f);
            }
    EXPECT(nf4_storage_bytes_ex(64, nullptr, 1), -1);

    // nf4_quantize
    auto q = [](const void *w, int dt, int64_t n, int bs, void *codes, void *am, int dq, void *aq,
                void *asc) {
        return nf4_quantize(w, (nf4_dtype)dt, n, bs, (uint8_t *)codes, (float *)am, dq,
                            (uint8_t *)aq, (float *)asc, nullptr);
    };
    EXPECT(q(F, 1, 0, 64, F, nullptr, 256, F, F), NF4_OK);
    EXPECT(q(F, 1, -1, 64, F, nullptr, 256, F, F), NF4_ERR_SIZE);
    EXPECT(q(F, 1, (int64_t(1) << 37) + 1, 64, F, nullptr, 256, F, F), NF4_ERR_SIZE);
    EXPECT(q(F, 1, 128, 32, F, nullptr, 256, F, F), NF4_ERR_UNSUPPORTED);
    EXPECT(q(F, 1, 128, 64, F, nullptr, 128, F, F), NF4_ERR_UNSUPPORTED);
    EXPECT(q(F, 7, 128, 64, F, nullptr, 256, F, F), NF4_ERR_UNSUPPORTED);
    EXPECT(q(nullptr, 1, 128, 64, F, nullptr, 256, F, F), NF4_ERR_NULL);
    EXPECT(q(F, 1, 128, 64, nullptr, nullptr, 256, F, F), NF4_ERR_NULL);
    EXPECT(q(F, 1, 128, 64, F, nullptr, 256, nullptr, F), NF4_ERR_NULL);
    EXPECT(q(F, 1, 128, 64, F, nullptr, 256, nullptr, nullptr), NF4_ERR_NULL);
    EXPECT(q(at<void>(8), 1, 128, 64, F, nullptr, 256, F, F), NF4_ERR_ALIGN);
    EXPECT(q(F, 1, 128, 64, at<void>(4), nullptr, 256, F, F), NF4_ERR_ALIGN);

    // nf4_double_quantize, nf4_dequantize
    EXPECT(nf4_double_quantize(at<float>(0), 0, 256, at<uint8_t>(0), at<float>(0), nullptr), NF4_OK);
    EXPECT(nf4_double_quantize(at<float>(0), -3, 256, at<uint8_t>(0), at<float>(0), nullptr), NF4_ERR_SIZE);
    EXPECT(nf4_double_quantize(at<float>(0), 10, 64, at<uint8_t>(0), at<float>(0), nullptr), NF4_ERR_UNSUPPORTED);
    EXPECT(nf4_double_quantize(nullptr, 10, 256, at<uint8_t>(0), at<float>(0), nullptr), NF4_ERR_NULL);
    EXPECT(nf4_double_quantize(at<float>(2), 10, 256, at<uint8_t>(0), at<float>(0), nullptr), NF4_ERR_ALIGN);
    EXPECT(nf4_dequantize(at<uint8_t>(0), 0, 64, nullptr, nullptr, nullptr, 256, F, NF4_BF16, nullptr), NF4_OK);
    EXPECT(nf4_dequantize(at<uint8_t>(0), 100, 64, nullptr, nullptr, nullptr, 256, F, NF4_BF16, nullptr),
           NF4_ERR_NULL);
    EXPECT(nf4_dequantize(at<uint8_t>(0), 100, 32, at<float>(0), nullptr, nullptr, 256, F, NF4_BF16, nullptr),
           NF4_ERR_UNSUPPORTED);
    EXPECT(nf4_dequantize(at<uint8_t>(0), 100, 64, at<float>(0), nullptr, nullptr, 256, at<void>(4), NF4_BF16,
                          nullptr), NF4_ERR_ALIGN);

    // batched calls: bad entries are reported before any launch
    nf4_batch_entry e[40];
    for (auto &x : e) x = nf4_batch_entry{F, 16384, at<uint8_t>(0), nullptr, at<uint8_t>(0), at<float>(0)};
    EXPECT(nf4_quantize_batched(e, 0, NF4_BF16, nullptr), NF4_OK);
    EXPECT(nf4_quantize_batched(nullptr, 3, NF4_BF16, nullptr), NF4_ERR_NULL);
    EXPECT(nf4_quantize_batched(e, -1, NF4_BF16, nullptr), NF4_ERR_SIZE);
    e[39].codes = nullptr;
    EXPECT(nf4_quantize_batched(e, 40, NF4_BF16, nullptr), NF4_ERR_NULL);
    e[39].codes = at<uint8_t>(0);
    e[17].w = at<void>(8);
    EXPECT(nf4_dequantize_batched(e, 40, NF4_BF16, nullptr), NF4_ERR_ALIGN);
    e[17].w = F;
    e[3].n = -5;
    EXPECT(nf4_quantize_batched(e, 40, NF4_F32, nullptr), NF4_ERR_SIZE);
    e[3].n = 16384;
    EXPECT(nf4_quantize_batched(e, 40, (nf4_dtype)9, nullptr), NF4_ERR_UNSUPPORTED);
}

void variants() {
    auto qx = [](const nf4_format *f, int64_t n, void *aq, void *off, void *ws, size_t wsb) {
        return nf4_quantize_ex(F, NF4_BF16, n, f, at<uint8_t>(0), nullptr, (uint8_t *)aq, at<float>(0),
                               (float *)off, ws, wsb, nullptr);
    };
    EXPECT(qx(nullptr, 1024, F, F, F, 1 << 20), NF4_ERR_NULL);
    for (const nf4_format &bad : {fmt(8), fmt(96), fmt(8192), fmt(64, 0), fmt(64, 3), fmt(64, 8192),
                                  fmt(64, 256, 3), fmt(64, 256, -1), fmt(64, 256, 0, 2),
                                  fmt(64, 256, 0, 0, 3), fmt(64, 256, 0, 0, -1)})
        EXPECT(qx(&bad, 1024, F, F, F, 1 << 20), NF4_ERR_UNSUPPORTED);
    const nf4_format d = fmt(), b128 = fmt(128), off = fmt(64, 256, 0, 1);
    EXPECT(qx(&d, -1, F, F, F, 1 << 20), NF4_ERR_SIZE);
    EXPECT(qx(&b128, 0, F, F, F, 1 << 20), NF4_OK);
    EXPECT(qx(&d, 1024, nullptr, F, F, 1 << 20), NF4_ERR_NULL);
    EXPECT(qx(&off, 1024, F, nullptr, F, 1 << 20), NF4_ERR_NULL);
    EXPECT(qx(&d, 1024, F, at<void>(2), F, 1 << 20), NF4_ERR_ALIGN);
    const size_t need = nf4_quantize_ex_workspace_size(1024, &b128);
    EXPECT(qx(&b128, 1024, F, F, nullptr, 1 << 20), NF4_ERR_WORKSPACE);
    EXPECT(qx(&b128, 1024, F, F, F, need - 1), NF4_ERR_WORKSPACE);
    EXPECT(qx(&b128, 1024, F, F, at<void>(16), 1 << 20), NF4_ERR_ALIGN);

    const nf4_format d5 = fmt(64, 5);
    EXPECT(nf4_double_quantize_ex(at<float>(0), 100, &d5, at<uint8_t>(0), at<float>(0), nullptr, nullptr, 0,
                                  nullptr), NF4_ERR_UNSUPPORTED);
    EXPECT(nf4_double_quantize_ex(at<float>(0), -1, &d, at<uint8_t>(0), at<float>(0), nullptr, nullptr, 0,
                                  nullptr), NF4_ERR_SIZE);
    EXPECT(nf4_double_quantize_ex(at<float>(0), 100, &off, at<uint8_t>(0), at<float>(0), at<float>(0), nullptr,
                                  0, nullptr), NF4_ERR_WORKSPACE);
    const nf4_format b32 = fmt(32), b32o = fmt(32, 256, 0, 1);
    EXPECT(nf4_dequantize_ex(at<uint8_t>(0), 1024, &b32, nullptr, at<uint8_t>(0), at<float>(0), nullptr, F,
                             (nf4_dtype)9, nullptr), NF4_ERR_UNSUPPORTED);
    EXPECT(nf4_dequantize_ex(at<uint8_t>(0), 1024, &b32o, nullptr, at<uint8_t>(0), at<float>(0), nullptr, F,
                             NF4_BF16, nullptr), NF4_ERR_NULL);
    EXPECT(nf4_dequantize_ex(at<uint8_t>(0), 0, &b32, nullptr, nullptr, nullptr, nullptr, nullptr, NF4_BF16,
                             nullptr), NF4_OK);
}

void linear() {
    const nf4_weight w = weight();
    const size_t ws = nf4_linear_workspace_size(64, 16);
    EXPECT(ws, 64 * 64 * 2 + 8 * 64 * 64 * 4);
    EXPECT(nf4_linear_workspace_size(100, 0), 0);
    for (auto fn : {nf4_linear_forward, nf4_linear_backward_input}) {
        EXPECT(fn(F, 64, nullptr, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_NULL);
        EXPECT(fn(F, 0, &w, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_OK);
        EXPECT(fn(F, -1, &w, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_SIZE);
        const nf4_weight k100 = weight(256, 100), bs32 = weight(256, 512, 32), dq64 = weight(256, 512, 64, 64);
        EXPECT(fn(F, 64, &k100, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_SIZE);
        EXPECT(fn(F, 64, &w, F, F, 300, 2.0f, F, F, ws, nullptr), NF4_ERR_SIZE);
        EXPECT(fn(F, 64, &bs32, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_UNSUPPORTED);
        EXPECT(fn(F, 64, &dq64, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_UNSUPPORTED);
        EXPECT(fn(nullptr, 64, &w, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_NULL);
        EXPECT(fn(F, 64, &w, nullptr, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_NULL);
        EXPECT(fn(at<void>(2), 64, &w, F, F, 16, 2.0f, F, F, ws, nullptr), NF4_ERR_ALIGN);
        EXPECT(fn(F, 64, &w, F, F, 16, 2.0f, F, nullptr, ws, nullptr), NF4_ERR_WORKSPACE);
        EXPECT(fn(F, 64, &w, F, F, 16, 2.0f, F, F, ws - 1, nullptr), NF4_ERR_WORKSPACE);
    }
    EXPECT(nf4_linear_forward_noalloc(F, 64, nullptr, F, F, 16, 2.0f, F, nullptr), NF4_ERR_NULL);
    EXPECT(nf4_linear_forward_noalloc(F, 0, &w, F, F, 16, 2.0f, F, nullptr), NF4_OK);
    EXPECT(nf4_linear_forward_noalloc(F, 4096, &w, F, F, 256, 2.0f, F, nullptr), NF4_ERR_SIZE);
    EXPECT(nf4_linear_forward_noalloc(at<void>(2), 64, &w, F, F, 16, 2.0f, F, nullptr), NF4_ERR_ALIGN);

    const size_t lws = nf4_lora_backward_workspace_size(64, 512, 256, 16);
    auto lb = [&](int64_t m, int64_t k, int64_t n, int r, void *ga, void *gb, int dt, void *wsp, size_t wsb) {
        return nf4_lora_backward(F, F, m, k, n, F, F, r, 2.0f, ga, gb, (nf4_dtype)dt, wsp, wsb, nullptr);
    };
    EXPECT(lb(-1, 512, 256, 16, F, F, 0, F, lws), NF4_ERR_SIZE);
    EXPECT(lb(64, 100, 256, 16, F, F, 0, F, lws), NF4_ERR_SIZE);
    EXPECT(lb(64, 512, 256, 12, F, F, 0, F, lws), NF4_ERR_SIZE);
    EXPECT(lb(64, 512, 256, 16, F, F, 7, F, lws), NF4_ERR_UNSUPPORTED);
    EXPECT(lb(64, 512, 256, 16, nullptr, nullptr, 0, F, lws), NF4_OK);
    EXPECT(lb(64, 512, 256, 16, F, F, 0, nullptr, lws), NF4_ERR_WORKSPACE);
    EXPECT(lb(64, 512, 256, 16, F, F, 0, F, lws - 1), NF4_ERR_WORKSPACE);
    EXPECT(lb(64, 512, 256, 16, F, F, 0, at<void>(16), lws), NF4_ERR_ALIGN);

    const size_t mws = nf4_merge_lora_workspace_size(256, 512);
    EXPECT(nf4_merge_lora(nullptr, F, F, 64, 2.0f, at<uint8_t>(0), nullptr, at<uint8_t>(0), at<float>(0), F,
                          mws, nullptr), NF4_ERR_NULL);
    EXPECT(nf4_merge_lora(&w, F, F, 64, 2.0f, at<uint8_t>(0), nullptr, nullptr, nullptr, F, mws, nullptr),
           NF4_ERR_NULL);
    EXPECT(nf4_merge_lora(&w, F, F, 64, 2.0f, at<uint8_t>(0), nullptr, at<uint8_t>(0), at<float>(0), nullptr,
                          mws, nullptr), NF4_ERR_WORKSPACE);
}

void code_tables() {
    // the bucket tables of the three codebooks build and pass their checks
    for (int cb = 0; cb < 3; ++cb) {
        const nf4::CodeLut *lut = nf4::code_lut_for(cb);
        EXPECT(lut != nullptr, 1);
        if (lut) EXPECT(lut->signmag, cb == NF4_CODEBOOK_FP4 ? 1 : 0);
    }
    EXPECT(nf4::code_lut_for(3) == nullptr, 1);
    EXPECT(nf4::code_lut_for(-1) == nullptr, 1);
    EXPECT(nf4::code_lut() == nf4::code_lut_for(NF4_CODEBOOK_NF4), 1);
}

}  // namespace

int main() {
    storage();
    variants();
    linear();
    code_tables();
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("host validation sanitizer run: ok\n");
    return 0;
}
