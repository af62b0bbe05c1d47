// Exercises the host side of the C ABI (include/ffn.h) without a GPU, for the
// AddressSanitizer / UndefinedBehaviorSanitizer build run by
// tests/test_sanitizers.py: the size queries over many shapes, the layout
// self-check, the kernel-family query, and every entry point with arguments
// that the host checks reject before any HIP call.  Exits non-zero on an unexpected return code.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ffn.h"

namespace {
int failures = 0;
void expect(int got, int want, const char* what) {
    if (got != want) {
        std::fprintf(stderr, "%s: got %d, want %d (%s)\n", what, got, want, ffn_last_error());
        ++failures;
    }
    if (want != FFN_OK && std::strlen(ffn_last_error()) == 0) {
        std::fprintf(stderr, "%s: no error text\n", what);
        ++failures;
    }
}
}  // namespace

int main() {
    if (ffn_version() < 100) return 1;
    if (ffn_selftest_layout() != 0) return 1;
    // size queries: valid and invalid shapes, every variant and form
    const int64_t dims[] = {-1, 0, 1, 7, 8, 16, 17, 64, 65, 448, 896, 1792, 4096, 8192, 1 << 20};
    size_t total = 0;
    for (int64_t M : dims)
        for (int64_t N : {8, 136, 4096})
            for (int64_t O : {8, 256, 448, 1792, 3584, 7168})
                for (int64_t P : {8, 520, 4096}) {
                    for (int dt = 0; dt < 3; ++dt)
                        for (int v = -1; v < 5; ++v) {
                            total += ffn_workspace_size_ex(M, N, O, P, dt, v);
                            total += ffn_swiglu_workspace_size(M, N, O, P, dt, v);
                        }
                    total += ffn_workspace_size(M, N, O, P, FFN_BF16);
                    total += ffn_backward_workspace_size(M, N, O, P, FFN_BF16);
                    for (int64_t E : {1, 8, 256, 257})
                        for (int k : {0, 1, 2, 8, 9}) total += moe_workspace_size(M, E, k, N, O, P, FFN_BF16);
                }
    if (total == 0) return 1;

    // rejected calls: fake, never dereferenced device pointers
    char* base = reinterpret_cast<char*>(0x100000);
    void* X = base;
    void* W = base + 0x1000;
    void* Y = base + 0x2000;
    void* ws = base + 0x10000;
    expect(ffn_forward(nullptr, W, nullptr, W, nullptr, Y, 64, 64, 448, 64, FFN_BF16, 2, 0, ws, 1 << 20, nullptr), FFN_EINVAL, "null X");
    expect(ffn_forward(X, W, nullptr, W, nullptr, Y, 64, 64, 12, 64, FFN_BF16, 2, 0, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "O % 8");
    expect(ffn_forward(X, W, nullptr, W, nullptr, Y, 64, 1 << 24, 8, 8, FFN_BF16, 2, 0, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "N bound");
    expect(ffn_forward(base + 8, W, nullptr, W, nullptr, Y, 64, 64, 448, 64, FFN_BF16, 2, 0, ws, 1 << 20, nullptr), FFN_EALIGN, "align");
    expect(ffn_forward(X, W, nullptr, W, nullptr, Y, 64, 64, 448, 64, FFN_BF16, 9, 0, ws, 1 << 20, nullptr), FFN_EINVAL, "act");
    expect(ffn_forward(X, W, nullptr, W, nullptr, Y, 64, 64, 448, 64, FFN_BF16, 2, 0, ws, 16, nullptr), FFN_EWORKSPACE, "workspace");
    expect(ffn_forward(X, W, nullptr, W, nullptr, Y, 0, 64, 448, 64, FFN_BF16, 2, 0, ws, 1 << 20, nullptr), FFN_OK, "M = 0");
    expect(ffn_forward_ex(X, W, nullptr, W, nullptr, Y, 17, 64, 448, 64, FFN_BF16, 2, 0, FFN_VARIANT_SKINNY, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "skinny M");
    void* evs[3] = {nullptr, nullptr, nullptr};
    expect(ffn_forward_traced(X, W, nullptr, W, nullptr, Y, 64, 64, 448, 64, FFN_BF16, 2, 0, 0, ws, 16, nullptr, evs, 2), FFN_EINVAL, "events");
    expect(ffn_forward_noalloc(X, W, nullptr, W, nullptr, Y, 4096, 4096, 1792, 4096, FFN_BF16, 2, 0, 0, nullptr), FFN_EWORKSPACE, "noalloc size");
    expect(ffn_swiglu_forward(X, W, nullptr, W, Y, 64, 64, 448, 64, FFN_BF16, 0, ws, 1 << 20, nullptr), FFN_EINVAL, "swiglu Wu");
    expect(ffn_swiglu_forward(X, W, W, W, Y, 64, 64, 448, 64, FFN_BF16, 0, ws, 16, nullptr), FFN_EWORKSPACE, "swiglu workspace");
    float* dW = reinterpret_cast<float*>(base + 0x3000);
    expect(ffn_backward(X, W, nullptr, W, Y, X, dW, nullptr, dW, nullptr, 64, 64, 64, 64, FFN_F32, 2, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "backward dtype");
    expect(ffn_backward(X, W, nullptr, W, Y, X, dW, nullptr, dW, nullptr, 64, 64, 64, 64, FFN_BF16, 2, ws, 16, nullptr), FFN_EWORKSPACE, "backward workspace");
    const float* lg = reinterpret_cast<const float*>(base + 0x4000);
    int32_t* ids = reinterpret_cast<int32_t*>(base + 0x5000);
    expect(moe_route(lg, 64, 8, 9, ids, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "route k");
    expect(moe_route(lg, 64, 300, 2, ids, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "route E");
    expect(moe_route(lg, 64, 8, 2, ids, nullptr, nullptr, nullptr, ws, 0, nullptr), FFN_EWORKSPACE, "route workspace");
    expect(moe_ffn_forward(X, nullptr, 64, 8, 2, W, nullptr, W, nullptr, Y, 64, 448, 64, FFN_BF16, 2, 0, nullptr, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr), FFN_EINVAL, "moe logits");
    expect(moe_ffn_forward(X, lg, 64, 8, 2, W, nullptr, W, nullptr, Y, 64, 448, 64, FFN_F32, 2, 0, nullptr, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "moe dtype");
    expect(moe_ffn_forward(X, lg, 64, 8, 2, W, nullptr, W, nullptr, Y, 64, 448, 64, FFN_BF16, 2, 0, nullptr, nullptr, nullptr, nullptr, ws, 16, nullptr), FFN_EWORKSPACE, "moe workspace");
    expect(moe_router(X, nullptr, nullptr, 64, 64, 8, 2, nullptr, ids, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr), FFN_EINVAL, "router Wr");
    expect(moe_router(X, W, nullptr, 64, 64, 12, 2, nullptr, ids, nullptr, nullptr, nullptr, ws, 1 << 20, nullptr), FFN_EUNSUPPORTED, "router E % 8");
    expect(moe_ffn_forward_router(X, W, nullptr, 64, 8, 2, W, nullptr, W, nullptr, Y, 64, 448, 64, FFN_BF16, 2, 0, nullptr, nullptr, nullptr, nullptr, nullptr, ws, 16, nullptr), FFN_EWORKSPACE, "moe router workspace");
    // the decode stream variant: shape and workspace checks, family queries
    expect(ffn_forward_ex(X, W, nullptr, W, nullptr, Y, 16, 4096, 1920, 4096, FFN_BF16, 2, 0, FFN_VARIANT_DECODE, ws, 1 << 30, nullptr), FFN_EUNSUPPORTED, "decode O");
    expect(ffn_forward_ex(X, W, nullptr, W, nullptr, Y, 16, 4096, 1792, 4096, FFN_BF16, 2, 0, FFN_VARIANT_DECODE, ws, 16, nullptr), FFN_EWORKSPACE, "decode workspace");
    expect(ffn_swiglu_forward(X, W, W, W, Y, 16, 4096, 1792, 8192, FFN_BF16, FFN_VARIANT_DECODE, ws, 1 << 30, nullptr), FFN_EUNSUPPORTED, "swiglu decode P");
    expect(ffn_selftest_decode_expiry(X, W, nullptr, W, nullptr, Y, 16, 1024, 896, 1024, 2, 0, ws, 1 << 30, nullptr), FFN_EUNSUPPORTED, "expiry shape");
    for (int v = 0; v < 5; ++v) {
        if (ffn_forward_family(16, 4096, 1792, 4096, FFN_BF16, v) < 0) return 1;
        if (ffn_forward_family(4096, 4096, 1792, 4096, FFN_BF16, v) < 0) return 1;
    }
    expect(ffn_forward_family(16, 4096, 1792, 4096, FFN_BF16, 7), FFN_EINVAL, "family variant");
    expect(ffn_forward_family(16, 4096, 12, 4096, FFN_BF16, 0), FFN_EUNSUPPORTED, "family shape");
    double flops = 0.0;
    expect(ffn_ceiling_mfma(ws, 0, 1, &flops, nullptr), FFN_EWORKSPACE, "ceiling sink");
    expect(ffn_ceiling_read(X, 24, ws, 1 << 20, nullptr), FFN_EINVAL, "ceiling bytes");
    if (failures) return 2;
    std::printf("api sanitizer driver: ok\n");
    return 0;
}
