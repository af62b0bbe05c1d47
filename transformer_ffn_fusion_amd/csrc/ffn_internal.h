// ffn_internal.h -- host-side launch interfaces between the C-ABI layer and
// the kernel translation units.  Not installed; the public interface is
// include/ffn.h.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <stddef.h>
#include <stdint.h>

namespace ffn {

// Raises a kernel's dynamic LDS limit on the current device, once per device
// (the attribute belongs to the device the call is made on).  `done` is the
// caller's per-kernel record; concurrent first calls both set the attribute,
// which is harmless.
constexpr int kMaxDevices = 64;
inline hipError_t set_dynamic_lds(const void* kern, int bytes,
                                  std::atomic<bool> (&done)[kMaxDevices]) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool known = dev >= 0 && dev < kMaxDevices;
    if (known && done[dev].load(std::memory_order_acquire)) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && known) done[dev].store(true, std::memory_order_release);
    return e;
}

// Sets the calling thread's error text (ffn_last_error) and returns `code`.
int set_error(int code, const char* fmt, ...);

// Compute units of the current device (queried once per device; 256 if the
// query fails).
inline int device_cus() {
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// ---- fused bf16 FFN with H kept in LDS (prefill shapes and the MoE groups)

constexpr int kPartBytes = 3;   // bytes of one packed split partial (16-bit significand)
constexpr int kBM = 64;     // token rows per workgroup tile
constexpr int kBN2 = 512;   // output columns per second-layer pass

// Hidden-chunk widths the fused kernel is instantiated for.
int fused_pick_chunk(int64_t O);                 // 256, 448 or 512
int fused_num_splits(int64_t O, int chunk);      // ceil(O / chunk)
int fused_pick_dense_chunk(int64_t M, int64_t O); // dense form: 896 (two passes) or fused_pick_chunk(O)

struct GroupedRows {
    const int32_t* tiles = nullptr;       // [max_tiles][3]: expert, first row, valid rows
    const int32_t* tile_count = nullptr;  // number of valid tiles (device)
    const int32_t* sorted = nullptr;      // sorted entries t*k+s; token = entry / k
    int k = 1;
    int64_t w1_stride = 0, w2_stride = 0, b1_stride = 0;  // per expert, in elements
};

// Writes packed partial outputs part[s][row][p] (kPartBytes each, s < splits)
// for rows < rows_out.
hipError_t launch_fused_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* b1,
                             const uint16_t* W2, void* part, int64_t M, int64_t N,
                             int64_t O, int64_t P, int act1, int chunk, int64_t row_blocks,
                             int64_t rows_out, const GroupedRows* grouped, hipStream_t stream);

// SwiGLU form: part[s][row][p] for the hidden chunk s of fused_swiglu_hid(O)
// columns: H = silu(X Wg) * (X Wu) rounded to bf16, times the rows of Wd.
int fused_swiglu_hid(int64_t O);                 // 448 or 256
int fused_swiglu_splits(int64_t O);              // ceil(O / fused_swiglu_hid(O))
hipError_t launch_fused_swiglu_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                    const uint16_t* Wd, void* part, int64_t M, int64_t N,
                                    int64_t O, int64_t P, hipStream_t stream);

// Y[m][p] = act2(sum_s part[s][m][p] + b2[p]) in ascending s; bf16 or fp32 out.
// The partials are packed (kPartBytes) with a bf16 output, fp32 with an fp32
// output (the fp32 path).
hipError_t launch_reduce_splits(const void* part, int splits, const void* b2, int b2_f32,
                                void* Y, int y_f32, int64_t M, int64_t P, int act2,
                                hipStream_t stream);

// ---- decode FFN (M <= 16) as one streaming kernel + one reduction, H
// exchanged inside each XCD's L2 (ffn_decode.hip).  Shapes: N = 4096,
// P = 4096, O a multiple of 256 up to 2048; a device of 256 CUs in 8 XCDs.
constexpr int64_t kDecodeN = 4096;
constexpr int64_t kDecodeP = 4096;
bool decode_stream_shape(int64_t M, int64_t N, int64_t O, int64_t P);
struct DecodeStreamLayout {   // workspace byte offsets, 256-byte aligned
    size_t part1, part1u, h, part2, flags, status, total;
};
DecodeStreamLayout decode_stream_layout(int64_t O, int64_t P, bool gated);
// W1u != nullptr: the gated (SwiGLU) form, W1 = Wg, W1u = Wu, W2 = Wd, no bias.
// expire: the self-test of the failure path (every wait expires, Y becomes NaN).
hipError_t launch_decode_stream(const uint16_t* X, const uint16_t* W1, const uint16_t* W1u,
                                const uint16_t* b1, const uint16_t* W2, char* ws, int64_t M,
                                int64_t O, int64_t P, int act1, uint64_t epoch,
                                hipStream_t stream, bool expire = false);
hipError_t launch_decode_reduce(const uint16_t* b2, uint16_t* Y, char* ws, int64_t M, int64_t O,
                                int64_t P, int act2, uint64_t epoch, bool gated,
                                hipStream_t stream);

// ---- skinny (M <= 16) bf16 layer with a fixed-order split-K reduction

constexpr int kSkinnyCols = 128;   // output columns per workgroup
constexpr int kSkinnyMaxM = 16;
int64_t skinny_kblock(int64_t K, int64_t Ncol);                 // rows of K per workgroup
size_t skinny_partial_floats(int64_t K, int64_t Ncol);          // workspace floats

// out[m][c] = act(sum_k A[m][k] W[k][c] + bias[c]) as bf16, m < M <= 16: a
// split-K weight-stream kernel plus an ordered reduction kernel.
hipError_t launch_skinny_bf16(const uint16_t* A, const uint16_t* W, const uint16_t* bias,
                              uint16_t* out, float* part, int64_t M, int64_t K, int64_t Ncol,
                              int act, hipStream_t stream);

// Gated first layer: out = bf16(silu(A Wg) * (A Wu)); both products write
// K-block partials (skinny_gated_partial_floats each), no bias.
size_t skinny_gated_partial_floats(int64_t K, int64_t Ncol);
hipError_t launch_skinny_swiglu_bf16(const uint16_t* A, const uint16_t* Wg, const uint16_t* Wu,
                                     uint16_t* out, float* part_g, float* part_u, int64_t M,
                                     int64_t K, int64_t Ncol, hipStream_t stream);

// ---- fp32 path

constexpr int kF32Chunk = 64;   // hidden columns per workgroup of the fp32 path
hipError_t launch_fused_f32(const float* X, const float* W1, const float* b1, const float* W2,
                            float* part, int64_t M, int64_t N, int64_t O, int64_t P, int act1,
                            hipStream_t stream);
hipError_t launch_fused_swiglu_f32(const float* X, const float* Wg, const float* Wu,
                                   const float* Wd, float* part, int64_t M, int64_t N, int64_t O,
                                   int64_t P, hipStream_t stream);

// ---- Mixture-of-Experts

int64_t moe_max_tiles(int64_t M, int64_t E, int k);

// Routing: top-k per token block (from the logits, or from X Wr + br when
// `logits` is null), then a one-workgroup scan (counts, offsets, block bases,
// tile table), then a parallel stable scatter into the per-expert lists.
struct RouteIO {
    const float* logits = nullptr;     // M x E fp32 gate logits, or null for the router form
    const uint16_t* X = nullptr;       // router form: M x N bf16
    const uint16_t* Wr = nullptr;      // router form: N x E bf16, E % 8 == 0
    const float* br = nullptr;         // router form: E fp32 or null
    float* logits_out = nullptr;       // router form: M x E fp32 or null
    int64_t M = 0, N = 0, E = 0;
    int k = 1;
    int32_t* ids = nullptr;            // M x k
    float* w = nullptr;                // M x k
    int32_t* counts = nullptr;         // E
    int32_t* offsets = nullptr;        // E + 1
    int32_t* sorted = nullptr;         // M x k
    int32_t* pos = nullptr;            // M x k
    int32_t* tiles = nullptr;          // moe_max_tiles x 3
    int32_t* tile_count = nullptr;     // 1
    int32_t* blk_counts = nullptr;     // moe_route_blocks_a x E
    int32_t* blk_base = nullptr;       // moe_route_blocks_b x E
};
int64_t moe_route_blocks_a(int64_t M, int64_t E, bool router);
int64_t moe_route_blocks_b(int64_t M);
hipError_t launch_moe_route(const RouteIO& io, hipStream_t stream);
hipError_t launch_moe_combine(const void* part, int splits, int64_t rows_total,
                              const int32_t* pos, const int32_t* ids, const float* w,
                              const uint16_t* b2, uint16_t* Y, int64_t M, int k, int64_t P,
                              int act2, hipStream_t stream);

// ---- backward (act2 none): recompute h and act1'(a), then five GEMMs and the
// bias column sums (ffn_backward.hip)

struct BackwardIO {
    const uint16_t *X = nullptr, *W1 = nullptr, *b1 = nullptr, *W2 = nullptr, *dY = nullptr;
    uint16_t* dX = nullptr;              // M x N bf16
    float *dW1 = nullptr, *db1 = nullptr, *dW2 = nullptr, *db2 = nullptr;
    uint16_t *H = nullptr, *Gr = nullptr, *dA = nullptr;   // workspace, M x O bf16 each
    float* colpart = nullptr;   // workspace, colsum_partial_floats(O, P) floats
    int64_t M = 0, N = 0, O = 0, P = 0;
    int act1 = 0;
};
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream);   // a fill kernel, no memset
size_t colsum_partial_floats(int64_t O, int64_t P);   // row-chunk partials of the bias sums
// events (may be null): events[s] recorded before step s + 1 (steps: h and g,
// da, dX, dW1, dW2, bias sums), events[6] after the last; n_events >= 7 to get all
hipError_t launch_ffn_backward(const BackwardIO& io, hipStream_t stream, void** events,
                               int n_events);

// ---- measurement support (ceilings.hip): the box's own MFMA and HBM ceilings

int ceiling_sink_floats();
hipError_t launch_ceiling_mfma(float* sink, int iters, double* flops, hipStream_t stream);
hipError_t launch_ceiling_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

}  // namespace ffn
