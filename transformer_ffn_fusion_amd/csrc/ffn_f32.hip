// ffn_f32.hip -- the fused FFN for fp32 inputs (small shapes, launch-bound).
//
// Same structure as the bf16 kernel (the kernel-fusion / tensor-parallelism
// post, brunomaga.github.io, section "Step 1: fusing the two linear layers"):
// a workgroup owns 8 token rows x a 64-wide chunk of the hidden dimension,
// computes that H tile with fp32 FMAs, applies b1 and the activation, keeps H
// in LDS and multiplies it by the matching rows of W2, writing an fp32 partial
// of Y per hidden chunk.  The shared split reduction adds b2 once and applies
// the second activation.  Everything stays fp32 (no rounding to bf16).
// The gated form (SwiGLU, same post, section "Benchmarks") accumulates the
// gate product X Wg and the up product X Wu side by side and keeps
// H = silu(gate) * up; it has no biases.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 8;                          // token rows per workgroup
constexpr int kKChunk = 256;                      // X columns staged in LDS at a time
constexpr int kKGroups = kThreads / kF32Chunk;    // layer 1: interleaved k-groups per column (4)
constexpr int kPTile = 128;                       // layer 2: output columns per sweep
constexpr int kOGroups = kThreads / kPTile;       // layer 2: hidden-row groups per column (2)
static_assert(kThreads % kF32Chunk == 0 && kThreads % kPTile == 0, "thread split");
static_assert(kF32Chunk % kOGroups == 0, "hidden rows split evenly");

// One workgroup = 8 rows x a 64-wide hidden chunk (many workgroups even for
// tiny shapes, so the dependent load chains of several chunks overlap).
// Layer 1: thread (g, c) sums k = g, g + 4, g + 8, ... for hidden column c;
// the four k-group sums are added in ascending g through LDS.  Layer 2:
// thread (h, p) sums hidden rows h*32 .. h*32+31 of the chunk for output
// column p; the two halves are added in ascending h.  Every sum has one
// fixed order, so results are bitwise reproducible.
template <bool kGated>
__global__ __launch_bounds__(kThreads) void fused_ffn_f32_kernel(
    const float* __restrict__ X, const float* __restrict__ W1, const float* __restrict__ W1u,
    const float* __restrict__ b1, const float* __restrict__ W2, float* __restrict__ part,
    int64_t M, int64_t N, int64_t O, int64_t P, int act1, int splits) {
    __shared__ float xs[kRows][kKChunk];
    __shared__ float red[kKGroups][kRows][kF32Chunk];
    __shared__ float redu[kGated ? kKGroups : 1][kRows][kF32Chunk];
    __shared__ float hs[kRows][kF32Chunk];
    __shared__ float ys[kOGroups][kRows][kPTile];

    const int tid = threadIdx.x;
    const int64_t rb = blockIdx.x / splits;
    const int s = (int)(blockIdx.x % splits);
    const int64_t row0 = rb * kRows;
    const int valid = (int)((M - row0) < kRows ? (M - row0) : kRows);
    const int64_t o0 = (int64_t)s * kF32Chunk;
    const int cl = tid % kF32Chunk;          // layer 1: hidden column of this thread
    const int kg = tid / kF32Chunk;          // ... and its k-group
    const int64_t o = o0 + cl;
    const bool ocol = o < O;

    float acc[kRows], accu[kRows];           // accu: the gated form's up product
#pragma unroll
    for (int r = 0; r < kRows; ++r) acc[r] = accu[r] = 0.f;
    for (int64_t k0 = 0; k0 < N; k0 += kKChunk) {
        for (int i = tid; i < kRows * kKChunk; i += kThreads) {
            const int r = i / kKChunk, kk = i % kKChunk;
            xs[r][kk] = (r < valid && k0 + kk < N) ? X[(row0 + r) * N + k0 + kk] : 0.f;
        }
        __syncthreads();
        const int kend = (N - k0) < kKChunk ? (int)(N - k0) : kKChunk;
        // unrolled so that many independent W1 loads are in flight at once
#pragma unroll 8
        for (int kk = kg; kk < kend; kk += kKGroups) {
            const float w = ocol ? W1[(k0 + kk) * O + o] : 0.f;
            float wu = 0.f;
            if constexpr (kGated) wu = ocol ? W1u[(k0 + kk) * O + o] : 0.f;
#pragma unroll
            for (int r = 0; r < kRows; ++r) {
                acc[r] = fmaf(xs[r][kk], w, acc[r]);
                if constexpr (kGated) accu[r] = fmaf(xs[r][kk], wu, accu[r]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        red[kg][r][cl] = acc[r];
        if constexpr (kGated) redu[kg][r][cl] = accu[r];
    }
    __syncthreads();
    if (tid < kF32Chunk) {
        const float bias = (ocol && b1) ? b1[o] : 0.f;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            float a = red[0][r][cl];
#pragma unroll
            for (int g = 1; g < kKGroups; ++g) a += red[g][r][cl];
            if constexpr (kGated) {
                float u = redu[0][r][cl];
#pragma unroll
                for (int g = 1; g < kKGroups; ++g) u += redu[g][r][cl];
                hs[r][cl] = ocol ? silu(a) * u : 0.f;
            } else {
                hs[r][cl] = ocol ? apply_act(act1, a + bias) : 0.f;
            }
        }
    }
    __syncthreads();

    // layer 2 partial: part[s][row0 + r][p] = sum_{o in chunk} H[r][o] W2[o][p]
    const int64_t oc = (O - o0) < kF32Chunk ? (O - o0) : kF32Chunk;
    constexpr int kOPer = kF32Chunk / kOGroups;
    const int og = tid / kPTile;
    const int pl = tid % kPTile;
    const int ob = og * kOPer;
    const int oe = (int)((ob + kOPer) < oc ? (ob + kOPer) : oc);
    float* dst = part + (int64_t)s * M * P;
    for (int64_t p0 = 0; p0 < P; p0 += kPTile) {
        const int64_t p = p0 + pl;
        float y[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) y[r] = 0.f;
        if (p < P) {
#pragma unroll 8
            for (int oo = ob; oo < oe; ++oo) {
                const float w = W2[(o0 + oo) * P + p];
#pragma unroll
                for (int r = 0; r < kRows; ++r) y[r] = fmaf(hs[r][oo], w, y[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < kRows; ++r) ys[og][r][pl] = y[r];
        __syncthreads();
        if (og == 0 && p < P) {
            for (int r = 0; r < valid; ++r) {
                float v = ys[0][r][pl];
#pragma unroll
                for (int g = 1; g < kOGroups; ++g) v += ys[g][r][pl];
                dst[(row0 + r) * P + p] = v;
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_fused_f32(const float* X, const float* W1, const float* b1, const float* W2,
                            float* part, int64_t M, int64_t N, int64_t O, int64_t P, int act1,
                            hipStream_t stream) {
    const int splits = (int)((O + kF32Chunk - 1) / kF32Chunk);
    const int64_t rbs = (M + kRows - 1) / kRows;
    if (rbs <= 0) return hipSuccess;
    hipLaunchKernelGGL(fused_ffn_f32_kernel<false>, dim3((unsigned)(rbs * splits)), dim3(kThreads),
                       0, stream, X, W1, nullptr, b1, W2, part, M, N, O, P, act1, splits);
    return hipGetLastError();
}

hipError_t launch_fused_swiglu_f32(const float* X, const float* Wg, const float* Wu,
                                   const float* Wd, float* part, int64_t M, int64_t N, int64_t O,
                                   int64_t P, hipStream_t stream) {
    const int splits = (int)((O + kF32Chunk - 1) / kF32Chunk);
    const int64_t rbs = (M + kRows - 1) / kRows;
    if (rbs <= 0) return hipSuccess;
    hipLaunchKernelGGL(fused_ffn_f32_kernel<true>, dim3((unsigned)(rbs * splits)), dim3(kThreads),
                       0, stream, X, Wg, Wu, nullptr, Wd, part, M, N, O, P, 0, splits);
    return hipGetLastError();
}

}  // namespace ffn
