// ffn_api.cpp -- the C ABI of libffn.so (declared in include/ffn.h): argument
// checks, workspace carving and dispatch to the gfx950 kernels.
//
// Every check that can fail runs on the host before the first launch, so a
// rejected call leaves all outputs untouched.  The library keeps no state
// between calls other than the error text of the calling host thread and the
// decode-stream call counter.
#include <hip/hip_runtime.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ffn.h"
#include "ffn_device.h"

#include "ffn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return FFN_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_act(int a) { return a == FFN_ACT_NONE || a == FFN_ACT_RELU || a == FFN_ACT_GELU_TANH; }

int check_dims(int64_t M, int64_t N, int64_t O, int64_t P) {
    if (M < 0) return fail(FFN_EINVAL, "M must be >= 0 (got %lld)", (long long)M);
    if (N < 1 || O < 1 || P < 1)
        return fail(FFN_EINVAL, "N, O, P must be >= 1 (got %lld, %lld, %lld)", (long long)N,
                    (long long)O, (long long)P);
    if (N % 8 || O % 8 || P % 8)
        return fail(FFN_EUNSUPPORTED, "N, O, P must be multiples of 8 (got %lld, %lld, %lld)",
                    (long long)N, (long long)O, (long long)P);
    const int64_t lim = (int64_t)1 << 31;
    if (M >= lim || N >= lim || O >= lim || P >= lim)
        return fail(FFN_EUNSUPPORTED, "dimensions must be below 2^31");
    // the kernels address each weight matrix with 32-bit byte offsets below 2^31
    if (N * O >= ((int64_t)1 << 30) || O * P >= ((int64_t)1 << 30))
        return fail(FFN_EUNSUPPORTED, "each weight matrix must hold fewer than 2^30 elements");
    // ... and a 64-row tile of X (fused kernel) or the up-to-16 rows of X and H
    // (decode layers, whose K is N or O) the same way: 64 * N * 2 and
    // 16 * O * 2 bytes below 2^31
    if (N >= ((int64_t)1 << 24) || O >= ((int64_t)1 << 24))
        return fail(FFN_EUNSUPPORTED, "N and O must be below 2^24 (got %lld, %lld)", (long long)N,
                    (long long)O);
    // ... and a 64-row tile of the packed split partials (64 * P * 3 bytes)
    if (P >= ((int64_t)1 << 23))
        return fail(FFN_EUNSUPPORTED, "P must be below 2^23 (got %lld)", (long long)P);
    return FFN_OK;
}

// A number that is new for every decode-stream call of this process (the
// call's flags in the workspace carry it, so they never need clearing); the
// start depends on the process's start time, so that another process's old
// flags in reused memory do not match either.
uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{
        (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() << 20};
    return counter.fetch_add(1, std::memory_order_relaxed) + 1;
}

int resolve_variant(int variant, int dtype, int64_t M) {
    if (variant == FFN_VARIANT_AUTO) {
        if (dtype == FFN_F32) return FFN_VARIANT_F32;
        return M <= ffn::kSkinnyMaxM ? FFN_VARIANT_SKINNY : FFN_VARIANT_FUSED;
    }
    return variant;
}

// ---- dense workspace layouts (byte offsets, each region 256-byte aligned)
struct DenseLayout {
    size_t part = 0;       // fused: packed partials; f32: fp32 partials
    size_t part1 = 0, h = 0, part2 = 0;
    size_t total = 0;
};

DenseLayout dense_layout(int64_t M, int64_t N, int64_t O, int64_t P, int variant) {
    DenseLayout L;
    if (variant == FFN_VARIANT_FUSED) {
        const int chunk = ffn::fused_pick_dense_chunk(M, O);
        const int S = ffn::fused_num_splits(O, chunk);
        L.part = 0;
        L.total = align_up((size_t)S * M * P * ffn::kPartBytes);
    } else if (variant == FFN_VARIANT_F32) {
        const int64_t S = (O + ffn::kF32Chunk - 1) / ffn::kF32Chunk;
        L.total = align_up((size_t)S * M * P * sizeof(float));
    } else if (variant == FFN_VARIANT_DECODE) {
        L.total = ffn::decode_stream_layout(O, P, false).total;
    } else {  // skinny; AUTO may run the decode stream instead, so the size covers both
        size_t off = 0;
        L.part1 = off;
        off += align_up(sizeof(float) * ffn::skinny_partial_floats(N, O));
        L.h = off;
        off += align_up(sizeof(uint16_t) * ffn::kSkinnyMaxM * O);
        L.part2 = off;
        off += align_up(sizeof(float) * ffn::skinny_partial_floats(O, P));
        L.total = off;
        if (ffn::decode_stream_shape(M, N, O, P)) {
            const size_t d = ffn::decode_stream_layout(O, P, false).total;
            if (d > L.total) L.total = d;
        }
    }
    if (L.total == 0) L.total = kAlign;
    return L;
}

// ---- SwiGLU workspace layouts
struct SwigluLayout {
    size_t part = 0;                          // fused: packed partials; f32: fp32 partials
    size_t part_g = 0, part_u = 0, h = 0, part2 = 0;  // skinny
    size_t total = 0;
};

SwigluLayout swiglu_layout(int64_t M, int64_t N, int64_t O, int64_t P, int variant) {
    SwigluLayout L;
    if (variant == FFN_VARIANT_FUSED) {
        L.total = align_up((size_t)ffn::fused_swiglu_splits(O) * M * P * ffn::kPartBytes);
    } else if (variant == FFN_VARIANT_F32) {
        const int64_t S = (O + ffn::kF32Chunk - 1) / ffn::kF32Chunk;
        L.total = align_up((size_t)S * M * P * sizeof(float));
    } else if (variant == FFN_VARIANT_DECODE) {
        L.total = ffn::decode_stream_layout(O, P, true).total;
    } else {  // skinny; AUTO may run the decode stream instead, so the size covers both
        size_t off = 0;
        L.part_g = off;
        off += align_up(sizeof(float) * ffn::skinny_gated_partial_floats(N, O));
        L.part_u = off;
        off += align_up(sizeof(float) * ffn::skinny_gated_partial_floats(N, O));
        L.h = off;
        off += align_up(sizeof(uint16_t) * ffn::kSkinnyMaxM * O);
        L.part2 = off;
        off += align_up(sizeof(float) * ffn::skinny_partial_floats(O, P));
        L.total = off;
        if (ffn::decode_stream_shape(M, N, O, P)) {
            const size_t d = ffn::decode_stream_layout(O, P, true).total;
            if (d > L.total) L.total = d;
        }
    }
    if (L.total == 0) L.total = kAlign;
    return L;
}

// ---- backward workspace layout
struct BackwardLayout {
    size_t H = 0, G = 0, dA = 0, colpart = 0, total = 0;
};

BackwardLayout backward_layout(int64_t M, int64_t O, int64_t P) {
    BackwardLayout L;
    size_t off = 0;
    L.H = off;       off += align_up(sizeof(uint16_t) * M * O);
    L.G = off;       off += align_up(sizeof(uint16_t) * M * O);
    L.dA = off;      off += align_up(sizeof(uint16_t) * M * O);
    L.colpart = off; off += align_up(sizeof(float) * ffn::colsum_partial_floats(O, P));
    L.total = off;
    return L;
}

// ---- MoE workspace layout
struct MoeLayout {
    size_t ids, w, counts, offsets, sorted, pos, tiles, tile_count, blk_counts, blk_base, part,
        total;
    int splits, chunk;
    int64_t max_tiles;
};

MoeLayout moe_layout(int64_t M, int64_t E, int k, int64_t O, int64_t P) {
    MoeLayout L{};
    const int64_t mk = M * k;
    L.chunk = ffn::fused_pick_chunk(O);
    L.splits = ffn::fused_num_splits(O, L.chunk);
    L.max_tiles = ffn::moe_max_tiles(M, E, k);
    size_t off = 0;
    L.ids = off;        off += align_up(sizeof(int32_t) * mk);
    L.w = off;          off += align_up(sizeof(float) * mk);
    L.counts = off;     off += align_up(sizeof(int32_t) * E);
    L.offsets = off;    off += align_up(sizeof(int32_t) * (E + 1));
    L.sorted = off;     off += align_up(sizeof(int32_t) * mk);
    L.pos = off;        off += align_up(sizeof(int32_t) * mk);
    L.tiles = off;      off += align_up(sizeof(int32_t) * 3 * (L.max_tiles + 1));
    L.tile_count = off; off += kAlign;
    // block histograms sized for the router form's 16-token blocks (the most blocks)
    L.blk_counts = off; off += align_up(sizeof(int32_t) * E * ffn::moe_route_blocks_a(M, E, true));
    L.blk_base = off;   off += align_up(sizeof(int32_t) * E * ffn::moe_route_blocks_b(M));
    L.part = off;       off += align_up((size_t)ffn::kPartBytes * L.splits * mk * P);
    L.total = off;
    return L;
}

int check_common_ptrs(const void* X, const void* W1, const void* b1, const void* W2,
                      const void* b2, const void* Y, void* ws, int64_t M) {
    // with M == 0 there are no rows: X and Y may be NULL (an empty tensor's pointer)
    if ((M > 0 && (!X || !Y)) || !W1 || !W2)
        return fail(FFN_EINVAL, "X, W1, W2 and Y must not be NULL");
    if (!ws) return fail(FFN_EINVAL, "workspace must not be NULL");
    const void* ps[] = {X, W1, b1, W2, b2, Y};
    const char* nm[] = {"X", "W1", "b1", "W2", "b2", "Y"};
    for (int i = 0; i < 6; ++i)
        if (ps[i] && !aligned16(ps[i])) return fail(FFN_EALIGN, "%s is not 16-byte aligned", nm[i]);
    if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
        return fail(FFN_EALIGN, "workspace is not 256-byte aligned");
    return FFN_OK;
}

int launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FFN_ELAUNCH, "%s: %s", what, hipGetErrorString(e));
    return FFN_OK;
}

}  // namespace

namespace ffn {
int set_error(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}
}  // namespace ffn

extern "C" {

int ffn_version(void) { return 100; }

const char* ffn_last_error(void) { return g_err; }

size_t ffn_workspace_size_ex(int64_t M, int64_t N, int64_t O, int64_t P, int dtype,
                             int variant) {
    if (check_dims(M, N, O, P) != FFN_OK) return 0;
    if (dtype != FFN_F32 && dtype != FFN_BF16) return 0;
    const int v = resolve_variant(variant, dtype, M);
    if (v < FFN_VARIANT_FUSED || v > FFN_VARIANT_DECODE) return 0;
    if (v == FFN_VARIANT_DECODE && (dtype != FFN_BF16 || !ffn::decode_stream_shape(M, N, O, P)))
        return 0;
    return dense_layout(M, N, O, P, v).total;
}

int ffn_forward_family(int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int variant) {
    int rc = check_dims(M, N, O, P);
    if (rc) return rc;
    if (dtype != FFN_F32 && dtype != FFN_BF16) return fail(FFN_EINVAL, "unknown dtype %d", dtype);
    if (variant < FFN_VARIANT_AUTO || variant > FFN_VARIANT_DECODE)
        return fail(FFN_EINVAL, "unknown variant %d", variant);
    const int v = resolve_variant(variant, dtype, M);
    if (variant == FFN_VARIANT_AUTO && v == FFN_VARIANT_SKINNY &&
        ffn::decode_stream_shape(M, N, O, P) && ffn::device_cus() == 256)
        return FFN_VARIANT_DECODE;
    return v;
}

size_t ffn_workspace_size(int64_t M, int64_t N, int64_t O, int64_t P, int dtype) {
    return ffn_workspace_size_ex(M, N, O, P, dtype, FFN_VARIANT_AUTO);
}

static int mark(void** events, int n_events, int i, hipStream_t st) {
    if (!events || i >= n_events) return FFN_OK;
    hipError_t e = hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), st);
    if (e != hipSuccess) return fail(FFN_ELAUNCH, "event record: %s", hipGetErrorString(e));
    return FFN_OK;
}

static int dense_forward(const void* X, const void* W1, const void* b1, const void* W2,
                         const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                         int dtype, int act1, int act2, int variant, void* workspace,
                         size_t workspace_bytes, void* stream, void** events, int n_events,
                         bool expire = false) {
    if (events && n_events < 3) return fail(FFN_EINVAL, "traced calls take at least 3 events");
    int rc = check_dims(M, N, O, P);
    if (rc) return rc;
    if (dtype != FFN_F32 && dtype != FFN_BF16) return fail(FFN_EINVAL, "unknown dtype %d", dtype);
    if (!valid_act(act1) || !valid_act(act2))
        return fail(FFN_EINVAL, "unknown activation (act1=%d, act2=%d)", act1, act2);
    if (variant < FFN_VARIANT_AUTO || variant > FFN_VARIANT_DECODE)
        return fail(FFN_EINVAL, "unknown variant %d", variant);
    rc = check_common_ptrs(X, W1, b1, W2, b2, Y, workspace, M);
    if (rc) return rc;
    const int v = resolve_variant(variant, dtype, M);
    if ((v == FFN_VARIANT_F32) != (dtype == FFN_F32))
        return fail(FFN_EUNSUPPORTED, "variant %d does not take dtype %d", v, dtype);
    if (v == FFN_VARIANT_SKINNY && M > ffn::kSkinnyMaxM)
        return fail(FFN_EUNSUPPORTED, "the skinny variant takes M <= %d (got %lld)",
                    ffn::kSkinnyMaxM, (long long)M);
    if (v == FFN_VARIANT_DECODE) {
        if (dtype != FFN_BF16 || !ffn::decode_stream_shape(M, N, O, P))
            return fail(FFN_EUNSUPPORTED,
                        "the decode variant takes bf16, M <= 16, N = P = 4096 and O a multiple "
                        "of 256 up to 2048 (got %lld x %lld x %lld x %lld)",
                        (long long)M, (long long)N, (long long)O, (long long)P);
        if (ffn::device_cus() != 256)
            return fail(FFN_EUNSUPPORTED, "the decode variant needs a device of 256 CUs (has %d)",
                        ffn::device_cus());
    }
    const DenseLayout L = dense_layout(M, N, O, P, v);
    if (workspace_bytes < L.total)
        return fail(FFN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    if (M == 0) return ok();

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    if ((rc = mark(events, n_events, 0, st))) return rc;
    if (v == FFN_VARIANT_FUSED) {
        const int chunk = ffn::fused_pick_dense_chunk(M, O);
        const int S = ffn::fused_num_splits(O, chunk);
        char* part = ws + L.part;
        const int64_t rbs = (M + ffn::kBM - 1) / ffn::kBM;
        rc = launched(ffn::launch_fused_bf16((const uint16_t*)X, (const uint16_t*)W1,
                                             (const uint16_t*)b1, (const uint16_t*)W2, part, M,
                                             N, O, P, act1, chunk, rbs, M, nullptr, st),
                      "fused FFN kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_reduce_splits(part, S, b2, 0, Y, 0, M, P, act2, st),
                      "split reduction kernel");
        if (rc) return rc;
    } else if (v == FFN_VARIANT_F32) {
        const int S = (int)((O + ffn::kF32Chunk - 1) / ffn::kF32Chunk);
        float* part = reinterpret_cast<float*>(ws + L.part);
        rc = launched(ffn::launch_fused_f32((const float*)X, (const float*)W1, (const float*)b1,
                                            (const float*)W2, part, M, N, O, P, act1, st),
                      "fp32 FFN kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_reduce_splits(part, S, b2, 1, Y, 1, M, P, act2, st),
                      "split reduction kernel");
        if (rc) return rc;
    } else if (ffn_forward_family(M, N, O, P, dtype, variant) == FFN_VARIANT_DECODE) {
        const uint64_t epoch = next_epoch();
        rc = launched(ffn::launch_decode_stream((const uint16_t*)X, (const uint16_t*)W1, nullptr,
                                                (const uint16_t*)b1, (const uint16_t*)W2, ws, M,
                                                O, P, act1, epoch, st, expire),
                      "decode streaming kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_decode_reduce((const uint16_t*)b2, (uint16_t*)Y, ws, M, O, P,
                                                act2, epoch, false, st),
                      "decode slice reduction");
        if (rc) return rc;
    } else {
        uint16_t* H = reinterpret_cast<uint16_t*>(ws + L.h);
        rc = launched(ffn::launch_skinny_bf16((const uint16_t*)X, (const uint16_t*)W1,
                                              (const uint16_t*)b1, H,
                                              reinterpret_cast<float*>(ws + L.part1), M, N, O,
                                              act1, st),
                      "skinny layer-1 kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_skinny_bf16(H, (const uint16_t*)W2, (const uint16_t*)b2,
                                              (uint16_t*)Y,
                                              reinterpret_cast<float*>(ws + L.part2), M, O, P,
                                              act2, st),
                      "skinny layer-2 kernel");
        if (rc) return rc;
    }
    if ((rc = mark(events, n_events, 2, st))) return rc;
    return ok();
}

int ffn_forward_ex(const void* X, const void* W1, const void* b1, const void* W2,
                   const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                   int dtype, int act1, int act2, int variant, void* workspace,
                   size_t workspace_bytes, void* stream) {
    return dense_forward(X, W1, b1, W2, b2, Y, M, N, O, P, dtype, act1, act2, variant, workspace,
                         workspace_bytes, stream, nullptr, 0);
}

int ffn_forward_traced(const void* X, const void* W1, const void* b1, const void* W2,
                       const void* b2, void* Y, int64_t M, int64_t N, int64_t O, int64_t P,
                       int dtype, int act1, int act2, int variant, void* workspace,
                       size_t workspace_bytes, void* stream, void** events, int n_events) {
    if (!events) return fail(FFN_EINVAL, "events must not be NULL");
    return dense_forward(X, W1, b1, W2, b2, Y, M, N, O, P, dtype, act1, act2, variant, workspace,
                         workspace_bytes, stream, events, n_events);
}

int ffn_forward(const void* X, const void* W1, const void* b1, const void* W2, const void* b2,
                void* Y, int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                int act2, void* workspace, size_t workspace_bytes, void* stream) {
    return ffn_forward_ex(X, W1, b1, W2, b2, Y, M, N, O, P, dtype, act1, act2,
                          FFN_VARIANT_AUTO, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- backward

size_t ffn_backward_workspace_size(int64_t M, int64_t N, int64_t O, int64_t P, int dtype) {
    if (check_dims(M, N, O, P) != FFN_OK || dtype != FFN_BF16) return 0;
    return backward_layout(M, O, P).total;
}

static int backward(const void* X, const void* W1, const void* b1, const void* W2,
                    const void* dY, void* dX, float* dW1, float* db1, float* dW2, float* db2,
                    int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                    void* workspace, size_t workspace_bytes, void* stream, void** events,
                    int n_events) {
    if (events && n_events < 7) return fail(FFN_EINVAL, "traced backward calls take at least 7 events");
    int rc = check_dims(M, N, O, P);
    if (rc) return rc;
    if (dtype != FFN_F32 && dtype != FFN_BF16) return fail(FFN_EINVAL, "unknown dtype %d", dtype);
    if (dtype != FFN_BF16) return fail(FFN_EUNSUPPORTED, "the backward takes bf16 only");
    if (!valid_act(act1)) return fail(FFN_EINVAL, "unknown activation %d", act1);
    if (!W1 || !W2 || !dW1 || !dW2 || (M > 0 && (!X || !dY || !dX)))
        return fail(FFN_EINVAL, "X, W1, W2, dY, dX, dW1 and dW2 must not be NULL");
    if (!workspace) return fail(FFN_EINVAL, "workspace must not be NULL");
    const void* ps[] = {X, W1, b1, W2, dY, dX, dW1, db1, dW2, db2};
    const char* nm[] = {"X", "W1", "b1", "W2", "dY", "dX", "dW1", "db1", "dW2", "db2"};
    for (int i = 0; i < 10; ++i)
        if (ps[i] && !aligned16(ps[i])) return fail(FFN_EALIGN, "%s is not 16-byte aligned", nm[i]);
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(FFN_EALIGN, "workspace is not 256-byte aligned");
    if (M * N >= ((int64_t)1 << 30) || M * O >= ((int64_t)1 << 30) || M * P >= ((int64_t)1 << 30))
        return fail(FFN_EUNSUPPORTED, "the backward addresses M x N, M x O and M x P with 32-bit "
                    "offsets: each must be below 2^30");
    const BackwardLayout L = backward_layout(M, O, P);
    if (workspace_bytes < L.total)
        return fail(FFN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (M == 0) {
        // no rows: every gradient is zero (a fill kernel: no memset nodes in a captured graph)
        const int64_t zn[4] = {N * O, O, O * P, P};
        float* zp[4] = {dW1, db1, dW2, db2};
        for (int i = 0; i < 4; ++i)
            if ((rc = launched(ffn::launch_zero_f32(zp[i], zn[i], st), "zero fill"))) return rc;
        return ok();
    }
    char* ws = static_cast<char*>(workspace);
    ffn::BackwardIO io;
    io.X = static_cast<const uint16_t*>(X);
    io.W1 = static_cast<const uint16_t*>(W1);
    io.b1 = static_cast<const uint16_t*>(b1);
    io.W2 = static_cast<const uint16_t*>(W2);
    io.dY = static_cast<const uint16_t*>(dY);
    io.dX = static_cast<uint16_t*>(dX);
    io.dW1 = dW1;
    io.db1 = db1;
    io.dW2 = dW2;
    io.db2 = db2;
    io.H = reinterpret_cast<uint16_t*>(ws + L.H);
    io.Gr = reinterpret_cast<uint16_t*>(ws + L.G);
    io.dA = reinterpret_cast<uint16_t*>(ws + L.dA);
    io.colpart = reinterpret_cast<float*>(ws + L.colpart);
    io.M = M;
    io.N = N;
    io.O = O;
    io.P = P;
    io.act1 = act1;
    rc = launched(ffn::launch_ffn_backward(io, st, events, n_events), "backward kernels");
    if (rc) return rc;
    return ok();
}

int ffn_backward(const void* X, const void* W1, const void* b1, const void* W2, const void* dY,
                 void* dX, float* dW1, float* db1, float* dW2, float* db2, int64_t M, int64_t N,
                 int64_t O, int64_t P, int dtype, int act1, void* workspace,
                 size_t workspace_bytes, void* stream) {
    return backward(X, W1, b1, W2, dY, dX, dW1, db1, dW2, db2, M, N, O, P, dtype, act1, workspace,
                    workspace_bytes, stream, nullptr, 0);
}

int ffn_backward_traced(const void* X, const void* W1, const void* b1, const void* W2,
                        const void* dY, void* dX, float* dW1, float* db1, float* dW2, float* db2,
                        int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                        void* workspace, size_t workspace_bytes, void* stream, void** events,
                        int n_events) {
    if (!events) return fail(FFN_EINVAL, "events must not be NULL");
    return backward(X, W1, b1, W2, dY, dX, dW1, db1, dW2, db2, M, N, O, P, dtype, act1, workspace,
                    workspace_bytes, stream, events, n_events);
}

// ---------------------------------------------------------------- SwiGLU

size_t ffn_swiglu_workspace_size(int64_t M, int64_t N, int64_t O, int64_t P, int dtype,
                                 int variant) {
    if (check_dims(M, N, O, P) != FFN_OK) return 0;
    if (dtype != FFN_F32 && dtype != FFN_BF16) return 0;
    const int v = resolve_variant(variant, dtype, M);
    if (v < FFN_VARIANT_FUSED || v > FFN_VARIANT_DECODE) return 0;
    if (v == FFN_VARIANT_DECODE && (dtype != FFN_BF16 || !ffn::decode_stream_shape(M, N, O, P)))
        return 0;
    return swiglu_layout(M, N, O, P, v).total;
}

static int swiglu_forward(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y,
                          int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int variant,
                          void* workspace, size_t workspace_bytes, void* stream, void** events,
                          int n_events) {
    if (events && n_events < 3) return fail(FFN_EINVAL, "traced calls take at least 3 events");
    int rc = check_dims(M, N, O, P);
    if (rc) return rc;
    if (dtype != FFN_F32 && dtype != FFN_BF16) return fail(FFN_EINVAL, "unknown dtype %d", dtype);
    if (variant < FFN_VARIANT_AUTO || variant > FFN_VARIANT_DECODE)
        return fail(FFN_EINVAL, "unknown variant %d", variant);
    if (!Wu) return fail(FFN_EINVAL, "Wu must not be NULL");
    if (!aligned16(Wu)) return fail(FFN_EALIGN, "Wu is not 16-byte aligned");
    rc = check_common_ptrs(X, Wg, nullptr, Wd, nullptr, Y, workspace, M);
    if (rc) return rc;
    const int v = resolve_variant(variant, dtype, M);
    if ((v == FFN_VARIANT_F32) != (dtype == FFN_F32))
        return fail(FFN_EUNSUPPORTED, "variant %d does not take dtype %d", v, dtype);
    if (v == FFN_VARIANT_SKINNY && M > ffn::kSkinnyMaxM)
        return fail(FFN_EUNSUPPORTED, "the skinny variant takes M <= %d (got %lld)",
                    ffn::kSkinnyMaxM, (long long)M);
    if (v == FFN_VARIANT_DECODE) {
        if (dtype != FFN_BF16 || !ffn::decode_stream_shape(M, N, O, P))
            return fail(FFN_EUNSUPPORTED,
                        "the decode variant takes bf16, M <= 16, N = P = 4096 and O a multiple "
                        "of 256 up to 2048 (got %lld x %lld x %lld x %lld)",
                        (long long)M, (long long)N, (long long)O, (long long)P);
        if (ffn::device_cus() != 256)
            return fail(FFN_EUNSUPPORTED, "the decode variant needs a device of 256 CUs (has %d)",
                        ffn::device_cus());
    }
    const SwigluLayout L = swiglu_layout(M, N, O, P, v);
    if (workspace_bytes < L.total)
        return fail(FFN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    if (M == 0) return ok();

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    if ((rc = mark(events, n_events, 0, st))) return rc;
    if (v == FFN_VARIANT_FUSED) {
        char* part = ws + L.part;   // packed partials
        rc = launched(ffn::launch_fused_swiglu_bf16((const uint16_t*)X, (const uint16_t*)Wg,
                                                    (const uint16_t*)Wu, (const uint16_t*)Wd, part,
                                                    M, N, O, P, st),
                      "fused SwiGLU kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_reduce_splits(part, ffn::fused_swiglu_splits(O), nullptr, 0, Y,
                                                0, M, P, FFN_ACT_NONE, st),
                      "split reduction kernel");
        if (rc) return rc;
    } else if (v == FFN_VARIANT_F32) {
        const int S = (int)((O + ffn::kF32Chunk - 1) / ffn::kF32Chunk);
        float* part = reinterpret_cast<float*>(ws + L.part);
        rc = launched(ffn::launch_fused_swiglu_f32((const float*)X, (const float*)Wg,
                                                   (const float*)Wu, (const float*)Wd, part, M, N,
                                                   O, P, st),
                      "fp32 SwiGLU kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_reduce_splits(part, S, nullptr, 1, Y, 1, M, P, FFN_ACT_NONE, st),
                      "split reduction kernel");
        if (rc) return rc;
    } else if (v == FFN_VARIANT_DECODE ||
               (variant == FFN_VARIANT_AUTO && ffn::decode_stream_shape(M, N, O, P) &&
                ffn::device_cus() == 256)) {
        const uint64_t epoch = next_epoch();
        rc = launched(ffn::launch_decode_stream((const uint16_t*)X, (const uint16_t*)Wg,
                                                (const uint16_t*)Wu, nullptr, (const uint16_t*)Wd,
                                                ws, M, O, P, FFN_ACT_NONE, epoch, st),
                      "gated decode streaming kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_decode_reduce(nullptr, (uint16_t*)Y, ws, M, O, P, FFN_ACT_NONE,
                                                epoch, true, st),
                      "decode slice reduction");
        if (rc) return rc;
    } else {
        uint16_t* H = reinterpret_cast<uint16_t*>(ws + L.h);
        rc = launched(ffn::launch_skinny_swiglu_bf16((const uint16_t*)X, (const uint16_t*)Wg,
                                                     (const uint16_t*)Wu, H,
                                                     reinterpret_cast<float*>(ws + L.part_g),
                                                     reinterpret_cast<float*>(ws + L.part_u), M,
                                                     N, O, st),
                      "skinny gated layer-1 kernel");
        if (rc) return rc;
        if ((rc = mark(events, n_events, 1, st))) return rc;
        rc = launched(ffn::launch_skinny_bf16(H, (const uint16_t*)Wd, nullptr, (uint16_t*)Y,
                                              reinterpret_cast<float*>(ws + L.part2), M, O, P,
                                              FFN_ACT_NONE, st),
                      "skinny layer-2 kernel");
        if (rc) return rc;
    }
    if ((rc = mark(events, n_events, 2, st))) return rc;
    return ok();
}

int ffn_swiglu_forward(const void* X, const void* Wg, const void* Wu, const void* Wd, void* Y,
                       int64_t M, int64_t N, int64_t O, int64_t P, int dtype, int variant,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return swiglu_forward(X, Wg, Wu, Wd, Y, M, N, O, P, dtype, variant, workspace,
                          workspace_bytes, stream, nullptr, 0);
}

int ffn_swiglu_forward_traced(const void* X, const void* Wg, const void* Wu, const void* Wd,
                              void* Y, int64_t M, int64_t N, int64_t O, int64_t P, int dtype,
                              int variant, void* workspace, size_t workspace_bytes, void* stream,
                              void** events, int n_events) {
    if (!events) return fail(FFN_EINVAL, "events must not be NULL");
    return swiglu_forward(X, Wg, Wu, Wd, Y, M, N, O, P, dtype, variant, workspace,
                          workspace_bytes, stream, events, n_events);
}

// ---------------------------------------------------------------- MoE

static int check_moe_dims(int64_t M, int64_t E, int k) {
    if (M < 0) return fail(FFN_EINVAL, "M must be >= 0");
    if (E < 1 || E > 256) return fail(FFN_EUNSUPPORTED, "E must be in [1, 256] (got %lld)", (long long)E);
    if (k < 1 || k > 8 || k > E)
        return fail(FFN_EUNSUPPORTED, "k must be in [1, min(E, 8)] (got %d)", k);
    if (M * k >= ((int64_t)1 << 31)) return fail(FFN_EUNSUPPORTED, "M*k must be below 2^31");
    return FFN_OK;
}

size_t moe_workspace_size(int64_t M, int64_t E, int k, int64_t N, int64_t O, int64_t P,
                          int dtype) {
    if (dtype != FFN_BF16) return 0;
    if (check_moe_dims(M, E, k) != FFN_OK) return 0;
    if (check_dims(M, N, O, P) != FFN_OK) return 0;
    return moe_layout(M, E, k, O, P).total;
}

// Routing into the workspace: from `logits`, or (logits == NULL) from the
// router X Wr + br, whose logits go to logits_out when it is not NULL.
static int route_into(const float* logits, const void* X, const void* Wr, const float* br,
                      float* logits_out, int64_t M, int64_t N, int64_t E, int k,
                      const MoeLayout& L, char* ws, int32_t** ids, float** w, hipStream_t st) {
    *ids = reinterpret_cast<int32_t*>(ws + L.ids);
    *w = reinterpret_cast<float*>(ws + L.w);
    ffn::RouteIO io;
    io.logits = logits;
    io.X = static_cast<const uint16_t*>(X);
    io.Wr = static_cast<const uint16_t*>(Wr);
    io.br = br;
    io.logits_out = logits ? nullptr : logits_out;
    io.M = M;
    io.N = N;
    io.E = E;
    io.k = k;
    io.ids = *ids;
    io.w = *w;
    io.counts = reinterpret_cast<int32_t*>(ws + L.counts);
    io.offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    io.sorted = reinterpret_cast<int32_t*>(ws + L.sorted);
    io.pos = reinterpret_cast<int32_t*>(ws + L.pos);
    io.tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
    io.tile_count = reinterpret_cast<int32_t*>(ws + L.tile_count);
    io.blk_counts = reinterpret_cast<int32_t*>(ws + L.blk_counts);
    io.blk_base = reinterpret_cast<int32_t*>(ws + L.blk_base);
    return launched(ffn::launch_moe_route(io, st), "routing kernels");
}

static int copy_route_outputs(int64_t M, int64_t E, int k, const MoeLayout& L, const char* ws,
                              int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                              int32_t* sorted_entries, hipStream_t st) {
    struct Cp { void* dst; size_t off, bytes; } cps[] = {
        {topk_ids, L.ids, sizeof(int32_t) * M * k},
        {topk_w, L.w, sizeof(float) * M * k},
        {expert_offsets, L.offsets, sizeof(int32_t) * (E + 1)},
        {sorted_entries, L.sorted, sizeof(int32_t) * M * k},
    };
    for (const Cp& c : cps) {
        if (!c.dst || c.bytes == 0) continue;
        hipError_t e = hipMemcpyAsync(c.dst, ws + c.off, c.bytes, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess) return fail(FFN_ELAUNCH, "routing output copy: %s", hipGetErrorString(e));
    }
    return FFN_OK;
}

int moe_route(const float* logits, int64_t M, int64_t E, int k, int32_t* topk_ids,
              float* topk_w, int32_t* expert_offsets, int32_t* sorted_entries,
              void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_moe_dims(M, E, k);
    if (rc) return rc;
    if (!logits || !workspace) return fail(FFN_EINVAL, "logits and workspace must not be NULL");
    if (reinterpret_cast<uintptr_t>(logits) & 3u) return fail(FFN_EALIGN, "logits not 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(FFN_EALIGN, "workspace is not 256-byte aligned");
    const MoeLayout L = moe_layout(M, E, k, 8, 8);
    if (workspace_bytes < L.part) return fail(FFN_EWORKSPACE, "workspace has %zu bytes, needs %zu",
                                              workspace_bytes, L.part);
    if (M == 0) return ok();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* ids;
    float* w;
    rc = route_into(logits, nullptr, nullptr, nullptr, nullptr, M, 0, E, k, L, ws, &ids, &w, st);
    if (rc) return rc;
    rc = copy_route_outputs(M, E, k, L, ws, topk_ids, topk_w, expert_offsets, sorted_entries, st);
    if (rc) return rc;
    return ok();
}

// Host checks of the router form's own arguments (X itself is checked by the caller).
static int check_router_args(const void* Wr, const float* br, const float* logits_out, int64_t E) {
    if (!Wr) return fail(FFN_EINVAL, "Wr must not be NULL");
    if (!aligned16(Wr)) return fail(FFN_EALIGN, "Wr is not 16-byte aligned");
    if (E % 8 != 0) return fail(FFN_EUNSUPPORTED, "the router form takes E a multiple of 8 (got %lld)", (long long)E);
    if (reinterpret_cast<uintptr_t>(br) & 3u) return fail(FFN_EALIGN, "br not 4-byte aligned");
    if (reinterpret_cast<uintptr_t>(logits_out) & 3u)
        return fail(FFN_EALIGN, "logits_out not 4-byte aligned");
    return FFN_OK;
}

// logits != NULL: routing from the given logits (Wr, br, logits_out unused);
// logits == NULL: the router form (logits = X Wr + br on the GPU).
static int moe_forward(const void* X, const float* logits, const void* Wr, const float* br,
                       float* logits_out, int64_t M, int64_t E, int k, const void* W1,
                       const void* b1, const void* W2, const void* b2, void* Y, int64_t N,
                       int64_t O, int64_t P, int dtype, int act1, int act2, int32_t* topk_ids,
                       float* topk_w, int32_t* expert_offsets, int32_t* sorted_entries,
                       void* workspace, size_t workspace_bytes, void* stream, void** events,
                       int n_events) {
    if (events && n_events < 4) return fail(FFN_EINVAL, "traced MoE calls take at least 4 events");
    int rc = check_moe_dims(M, E, k);
    if (rc) return rc;
    rc = check_dims(M, N, O, P);
    if (rc) return rc;
    if (dtype != FFN_BF16) return fail(FFN_EUNSUPPORTED, "the grouped form takes bf16 only");
    if (!valid_act(act1) || !valid_act(act2))
        return fail(FFN_EINVAL, "unknown activation (act1=%d, act2=%d)", act1, act2);
    if (logits) {
        if (reinterpret_cast<uintptr_t>(logits) & 3u) return fail(FFN_EALIGN, "logits not 4-byte aligned");
    } else {
        rc = check_router_args(Wr, br, logits_out, E);
        if (rc) return rc;
    }
    rc = check_common_ptrs(X, W1, b1, W2, b2, Y, workspace, M);
    if (rc) return rc;
    if (M * N >= ((int64_t)1 << 30))
        return fail(FFN_EUNSUPPORTED, "the grouped form gathers from X with 32-bit offsets: M*N < 2^30");
    const MoeLayout L = moe_layout(M, E, k, O, P);
    if (workspace_bytes < L.total)
        return fail(FFN_EWORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, L.total);
    if (M == 0) return ok();

    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* ids;
    float* w;
    if ((rc = mark(events, n_events, 0, st))) return rc;
    rc = route_into(logits, X, Wr, br, logits_out, M, N, E, k, L, ws, &ids, &w, st);
    if (rc) return rc;
    if ((rc = mark(events, n_events, 1, st))) return rc;

    ffn::GroupedRows g;
    g.tiles = reinterpret_cast<const int32_t*>(ws + L.tiles);
    g.tile_count = reinterpret_cast<const int32_t*>(ws + L.tile_count);
    g.sorted = reinterpret_cast<const int32_t*>(ws + L.sorted);
    g.k = k;
    g.w1_stride = N * O;
    g.w2_stride = O * P;
    g.b1_stride = O;
    const int64_t row_blocks = (L.max_tiles + 7) / 8 * 8;
    char* part = ws + L.part;   // packed partials
    rc = launched(ffn::launch_fused_bf16((const uint16_t*)X, (const uint16_t*)W1,
                                         (const uint16_t*)b1, (const uint16_t*)W2, part, M, N, O,
                                         P, act1, L.chunk, row_blocks, M * k, &g, st),
                  "grouped FFN kernel");
    if (rc) return rc;
    if ((rc = mark(events, n_events, 2, st))) return rc;
    rc = launched(ffn::launch_moe_combine(part, L.splits, M * k,
                                          reinterpret_cast<const int32_t*>(ws + L.pos), ids, w,
                                          (const uint16_t*)b2, (uint16_t*)Y, M, k, P, act2, st),
                  "combine kernel");
    if (rc) return rc;
    if ((rc = mark(events, n_events, 3, st))) return rc;
    rc = copy_route_outputs(M, E, k, L, ws, topk_ids, topk_w, expert_offsets, sorted_entries, st);
    if (rc) return rc;
    return ok();
}

int moe_ffn_forward(const void* X, const float* logits, int64_t M, int64_t E, int k,
                    const void* W1, const void* b1, const void* W2, const void* b2, void* Y,
                    int64_t N, int64_t O, int64_t P, int dtype, int act1, int act2,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                    int32_t* sorted_entries, void* workspace, size_t workspace_bytes,
                    void* stream) {
    if (!logits) return fail(FFN_EINVAL, "logits must not be NULL");
    return moe_forward(X, logits, nullptr, nullptr, nullptr, M, E, k, W1, b1, W2, b2, Y, N, O, P,
                       dtype, act1, act2, topk_ids, topk_w, expert_offsets, sorted_entries,
                       workspace, workspace_bytes, stream, nullptr, 0);
}

int moe_ffn_forward_router(const void* X, const void* Wr, const float* br, int64_t M, int64_t E,
                           int k, const void* W1, const void* b1, const void* W2, const void* b2,
                           void* Y, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                           int act2, float* logits_out, int32_t* topk_ids, float* topk_w,
                           int32_t* expert_offsets, int32_t* sorted_entries, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return moe_forward(X, nullptr, Wr, br, logits_out, M, E, k, W1, b1, W2, b2, Y, N, O, P, dtype,
                       act1, act2, topk_ids, topk_w, expert_offsets, sorted_entries, workspace,
                       workspace_bytes, stream, nullptr, 0);
}

int moe_router(const void* X, const void* Wr, const float* br, int64_t M, int64_t N, int64_t E,
               int k, float* logits_out, int32_t* topk_ids, float* topk_w,
               int32_t* expert_offsets, int32_t* sorted_entries, void* workspace,
               size_t workspace_bytes, void* stream) {
    int rc = check_moe_dims(M, E, k);
    if (rc) return rc;
    if (N < 8 || N % 8 != 0) return fail(FFN_EUNSUPPORTED, "N must be a positive multiple of 8");
    if ((M > 0 && !X) || !workspace) return fail(FFN_EINVAL, "X and workspace must not be NULL");
    if (X && !aligned16(X)) return fail(FFN_EALIGN, "X is not 16-byte aligned");
    rc = check_router_args(Wr, br, logits_out, E);
    if (rc) return rc;
    if (reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1))
        return fail(FFN_EALIGN, "workspace is not 256-byte aligned");
    const MoeLayout L = moe_layout(M, E, k, 8, 8);
    if (workspace_bytes < L.part) return fail(FFN_EWORKSPACE, "workspace has %zu bytes, needs %zu",
                                              workspace_bytes, L.part);
    if (M == 0) return ok();
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* ids;
    float* w;
    rc = route_into(nullptr, X, Wr, br, logits_out, M, N, E, k, L, ws, &ids, &w, st);
    if (rc) return rc;
    rc = copy_route_outputs(M, E, k, L, ws, topk_ids, topk_w, expert_offsets, sorted_entries, st);
    if (rc) return rc;
    return ok();
}

int moe_ffn_forward_traced(const void* X, const float* logits, int64_t M, int64_t E, int k,
                           const void* W1, const void* b1, const void* W2, const void* b2,
                           void* Y, int64_t N, int64_t O, int64_t P, int dtype, int act1,
                           int act2, void* workspace, size_t workspace_bytes, void* stream,
                           void** events, int n_events) {
    if (!events) return fail(FFN_EINVAL, "events must not be NULL");
    if (!logits) return fail(FFN_EINVAL, "logits must not be NULL");
    return moe_forward(X, logits, nullptr, nullptr, nullptr, M, E, k, W1, b1, W2, b2, Y, N, O, P,
                       dtype, act1, act2, nullptr, nullptr, nullptr, nullptr, workspace,
                       workspace_bytes, stream, events, n_events);
}

// ---------------------------------------------------------------- self-check

size_t ffn_ceiling_sink_bytes(void) { return (size_t)ffn::ceiling_sink_floats() * 4; }

int ffn_ceiling_mfma(void* sink, size_t sink_bytes, int iters, double* flops_per_launch,
                     void* stream) {
    if (!sink || !flops_per_launch) return fail(FFN_EINVAL, "sink and flops_per_launch must not be NULL");
    if (sink_bytes < ffn_ceiling_sink_bytes())
        return fail(FFN_EWORKSPACE, "sink has %zu bytes, needs %zu", sink_bytes, ffn_ceiling_sink_bytes());
    if (iters < 1) return fail(FFN_EINVAL, "iters must be >= 1 (got %d)", iters);
    double f = 0.0;
    int rc = launched(ffn::launch_ceiling_mfma(static_cast<float*>(sink), iters, &f,
                                               reinterpret_cast<hipStream_t>(stream)),
                      "MFMA ceiling kernel");
    if (rc) return rc;
    *flops_per_launch = f;
    return ok();
}

int ffn_ceiling_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream) {
    if (!src || !sink) return fail(FFN_EINVAL, "src and sink must not be NULL");
    if (!aligned16(src)) return fail(FFN_EALIGN, "src not 16-byte aligned");
    if (bytes < 16 || bytes % 16) return fail(FFN_EINVAL, "bytes must be a positive multiple of 16");
    if (sink_bytes < ffn_ceiling_sink_bytes())
        return fail(FFN_EWORKSPACE, "sink has %zu bytes, needs %zu", sink_bytes, ffn_ceiling_sink_bytes());
    int rc = launched(ffn::launch_ceiling_read(src, bytes, static_cast<uint32_t*>(sink),
                                               reinterpret_cast<hipStream_t>(stream)),
                      "read ceiling kernel");
    return rc ? rc : ok();
}

int ffn_selftest_decode_expiry(const void* X, const void* W1, const void* b1, const void* W2,
                               const void* b2, void* Y, int64_t M, int64_t N, int64_t O,
                               int64_t P, int act1, int act2, void* workspace,
                               size_t workspace_bytes, void* stream) {
    return dense_forward(X, W1, b1, W2, b2, Y, M, N, O, P, FFN_BF16, act1, act2,
                         FFN_VARIANT_DECODE, workspace, workspace_bytes, stream, nullptr, 0, true);
}

int ffn_selftest_layout(void) {
    // Fragment reads: for each 16-index fragment and k-group, the 16 lanes hit
    // 16 distinct 16-byte slots of one 256-byte line (and 8 distinct slots in
    // each half-wave group of 8 lanes, for 32-bank hardware).
    for (uint32_t f = 0; f < 64; ++f) {
        for (uint32_t g = 0; g < 4; ++g) {
            uint32_t seen16 = 0, line = ~0u;
            for (uint32_t i = 0; i < 16; ++i) {
                uint32_t off = ffn::frag_off(16 * f + i, g);
                if (line == ~0u) line = off >> 8;
                if ((off >> 8) != line) return 1;
                seen16 |= 1u << ((off >> 4) & 15);
            }
            if (seen16 != 0xffffu) return 2;
            for (uint32_t h = 0; h < 2; ++h) {
                uint32_t seen8 = 0;
                for (uint32_t i = 0; i < 8; ++i)
                    seen8 |= 1u << ((ffn::frag_off(16 * f + 8 * h + i, g) >> 4) & 7);
                if (seen8 != 0xffu) return 3;
            }
        }
    }
    // The offsets of one tile are a bijection onto [0, 64 * idx_count).
    static unsigned char hit[64 * 512];
    std::memset(hit, 0, sizeof hit);
    for (uint32_t idx = 0; idx < 512; ++idx)
        for (uint32_t g = 0; g < 4; ++g) {
            uint32_t off = ffn::frag_off(idx, g);
            if (off % 16 || off / 16 >= 4 * 512 || hit[off / 16]) return 6;
            hit[off / 16] = 1;
        }

    // Weight stage blocks (8 k-rows x 64 columns, 1 KiB), filled by lane l of a
    // direct-to-LDS load writing slot l.  slot -> (row, 8-column group) it holds:
    auto wslot_row = [](uint32_t slot) { return slot >> 3; };
    auto wslot_grp = [](uint32_t slot) { return (slot & 7) ^ ((2 * (slot >> 3)) & 7); };
    const uint32_t rb = 4096;   // a row pitch larger than any in-row offset
    for (uint32_t l = 0; l < 64; ++l) {
        const uint32_t off = ffn::wtile_dma_off((int)l, rb);
        if (off / rb != wslot_row(l) || (off % rb) % 16 || (off % rb) / 16 != wslot_grp(l)) return 7;
    }
    for (uint32_t q0 = 0; q0 < 64; q0 += 4) {   // each lane quad reads one 64-byte segment
        const uint32_t seg = ffn::wtile_dma_off((int)q0, rb) / 64;
        for (uint32_t l = q0; l < q0 + 4; ++l)
            if (ffn::wtile_dma_off((int)l, rb) / 64 != seg) return 8;
    }
    // Transposing reads: lane l (g = l/16, j = (l%16)/4, q = l%4) of the read
    // for fragment f, half t must address row 8g + j + 4t, column group 2f + q/2,
    // 4-column half q%2; the 16 lanes of a group (4 rows) hit 16 distinct
    // 8-byte bank positions modulo 128 bytes.
    for (int nb = 7; nb <= 8; ++nb)
        for (int f = 0; f < 4 * nb; ++f)
            for (int t = 0; t < 2; ++t) {
                for (int g0 = 0; g0 < 64; g0 += 16) {
                    uint32_t seen = 0;
                    for (int l = g0; l < g0 + 16; ++l) {
                        const uint32_t off = ffn::wtile_tr_base(l, nb, f % 4) + 1024u * (f / 4) + 512u * t;
                        const uint32_t g = l >> 4, j = (l & 15) >> 2, q = l & 3;
                        const uint32_t c8 = 2 * f + (q >> 1);
                        const uint32_t blk = off / 1024, slot = (off % 1024) / 16;
                        if (blk != g * nb + (c8 >> 3)) return 9;
                        if (wslot_row(slot) != j + 4 * t || wslot_grp(slot) != (c8 & 7)) return 10;
                        if ((off % 16) / 8 != (q & 1) || off % 8) return 11;
                        seen |= 1u << ((off % 128) / 8);
                    }
                    if (seen != 0xffffu) return 13;
                }
            }
    // X fragments (16 rows x 32 k): lane l of the load writes slot l = row l/4,
    // k-group (l%4) ^ (l/8 mod 4); the operand read of lane l (row l%16,
    // k-group l/16) must find that unit, conflict-free in every 8-lane group.
    for (int l = 0; l < 64; ++l) {
        const int r = l >> 2, c = (l & 3) ^ ((l >> 3) & 3);
        if (ffn::xfrag_slot(r, c) != l) return 14;
    }
    uint64_t all = 0;
    for (int g0 = 0; g0 < 64; g0 += 8) {
        uint32_t seen = 0;
        for (int l = g0; l < g0 + 8; ++l) {
            const int slot = ffn::xfrag_slot(l & 15, l >> 4);
            seen |= 1u << (slot & 7);
            all |= 1ull << slot;
        }
        if (seen != 0xffu) return 15;
    }
    if (all != ~0ull) return 16;
    return 0;
}

}  // extern "C"
