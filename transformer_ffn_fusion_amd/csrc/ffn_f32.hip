// ffn_f32.hip -- the fused FFN for fp32 inputs (small shapes, launch-bound).
//
// Same structure as the bf16 kernel (the kernel-fusion / tensor-parallelism
// post, brunomaga.github.io, section "Step 1: fusing the two linear layers"):
// a workgroup owns 8 token rows x a 512-wide chunk of the hidden dimension,
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
constexpr int kRows = 8;
constexpr int kKChunk = 256;
constexpr int kColsPerThread = kF32Chunk / kThreads;  // 2

template <bool kGated>
__global__ __launch_bounds__(kThreads) void fused_ffn_f32_kernel(
    const float* __restrict__ X, const float* __restrict__ W1, const float* __restrict__ W1u,
    const float* __restrict__ b1, const float* __restrict__ W2, float* __restrict__ part,
    int64_t M, int64_t N, int64_t O, int64_t P, int act1, int splits) {
    __shared__ float xs[kRows][kKChunk];
    __shared__ float hs[kRows][kF32Chunk];

    const int tid = threadIdx.x;
    const int64_t rb = blockIdx.x / splits;
    const int s = (int)(blockIdx.x % splits);
    const int64_t row0 = rb * kRows;
    const int valid = (int)((M - row0) < kRows ? (M - row0) : kRows);
    const int64_t o0 = (int64_t)s * kF32Chunk;

    float acc[kRows][kColsPerThread];
    float accu[kRows][kColsPerThread];   // gated form: the up product
#pragma unroll
    for (int r = 0; r < kRows; ++r)
#pragma unroll
        for (int j = 0; j < kColsPerThread; ++j) acc[r][j] = accu[r][j] = 0.f;

    // layer 1: acc[r][j] = sum_n X[row0 + r][n] W1[n][o0 + tid + 256 j]
    for (int64_t k0 = 0; k0 < N; k0 += kKChunk) {
        for (int i = tid; i < kRows * kKChunk; i += kThreads) {
            const int r = i / kKChunk, kk = i % kKChunk;
            xs[r][kk] = (r < valid && k0 + kk < N) ? X[(row0 + r) * N + k0 + kk] : 0.f;
        }
        __syncthreads();
        const int kend = (N - k0) < kKChunk ? (int)(N - k0) : kKChunk;
        // unrolled so that many independent W1 loads are in flight at once
#pragma unroll 16
        for (int kk = 0; kk < kend; ++kk) {
            float w[kColsPerThread], wu[kColsPerThread];
#pragma unroll
            for (int j = 0; j < kColsPerThread; ++j) {
                const int64_t o = o0 + tid + kThreads * j;
                w[j] = o < O ? W1[(k0 + kk) * O + o] : 0.f;
                if constexpr (kGated) wu[j] = o < O ? W1u[(k0 + kk) * O + o] : 0.f;
            }
#pragma unroll
            for (int r = 0; r < kRows; ++r)
#pragma unroll
                for (int j = 0; j < kColsPerThread; ++j) {
                    acc[r][j] = fmaf(xs[r][kk], w[j], acc[r][j]);
                    if constexpr (kGated) accu[r][j] = fmaf(xs[r][kk], wu[j], accu[r][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < kColsPerThread; ++j) {
        const int ol = tid + kThreads * j;
        const int64_t o = o0 + ol;
        const float bias = (o < O && b1) ? b1[o] : 0.f;
#pragma unroll
        for (int r = 0; r < kRows; ++r) {
            if constexpr (kGated)
                hs[r][ol] = o < O ? silu(acc[r][j]) * accu[r][j] : 0.f;
            else
                hs[r][ol] = o < O ? apply_act(act1, acc[r][j] + bias) : 0.f;
        }
    }
    __syncthreads();

    // layer 2 partial: part[s][row0 + r][p] = sum_{o in chunk} H[r][o] W2[o][p]
    const int64_t oc = (O - o0) < kF32Chunk ? (O - o0) : kF32Chunk;
    float* dst = part + (int64_t)s * M * P;
    for (int64_t p = tid; p < P; p += kThreads) {
        float y[kRows];
#pragma unroll
        for (int r = 0; r < kRows; ++r) y[r] = 0.f;
#pragma unroll 16
        for (int o = 0; o < (int)oc; ++o) {
            const float w = W2[(o0 + o) * P + p];
#pragma unroll
            for (int r = 0; r < kRows; ++r) y[r] = fmaf(hs[r][o], w, y[r]);
        }
        for (int r = 0; r < valid; ++r) dst[(row0 + r) * P + p] = y[r];
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
