// ffn_skinny.hip -- one FFN layer for decode-sized batches (M <= 16 rows).
//
// out[m][c] = act( sum_k A[m][k] W[k][c] + bias[c] ), bf16 in and out, fp32
// accumulation.  Called twice per FFN: layer 1 (A = X, W = W1, bias = b1,
// act = act1 -> H) and layer 2 (A = H, W = W2, bias = b2, act = act2 -> Y),
// following the two equations of the kernel-fusion / tensor-parallelism post
// (brunomaga.github.io), section "Megatron-LM tensor parallelism".
//
// At M = 16 the layer is a weight stream: every byte of W is used for 16 rows
// only, so the time is the HBM time of W.  The design is built for that:
//  * one workgroup owns 128 output columns x a block of K rows of W; every
//    lane issues all of its 16-byte weight loads before any math, so the whole
//    weight matrix is in flight at once across the grid;
//  * the 16 rows map exactly onto the 16-row side of v_mfma_f32_16x16x32_bf16;
//    the weight block is transposed in registers (8x8 per lane) straight into
//    the MFMA operand layout -- no LDS round trip for the weights;
//  * the K blocks are reduced in a fixed order by a second small kernel: each
//    workgroup writes its fp32 partial; the reduction sums them in ascending
//    K-block order, adds the bias once, applies the activation and rounds once
//    to bf16.  (A last-arriver reduction inside the first kernel would need a
//    device-scope release per workgroup; on this part that fence writes back
//    the XCD's L2 and the workgroups of an XCD serialise on it -- measured at
//    ~20 us per layer, against ~1.5 us for the loads and the math.)
//
// Gated first layer (SwiGLU: same post, section "Benchmarks"): the grid gets a
// second z-slice that streams the up matrix Wu beside the gate matrix Wg, both
// slices always write partials, and the reduction forms
// H = silu(sum gate) * (sum up) before its single rounding to bf16.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;    // a reduction thread keeps 2 * kBatch K-block partial loads in flight

struct SkinnyArgs {
    const uint16_t* A;
    const uint16_t* W;
    const uint16_t* Wu;   // gated: the up matrix (grid z-slice 1)
    const uint16_t* bias;
    uint16_t* out;
    float* part;        // [nkb][16][Ncol]
    float* part_u;      // gated: partials of the up product
    int64_t M, K, Ncol;
    int64_t kblock;
    int nkb;
    int act;
    int gated;
};

template <int KSTEPS>
__global__ __launch_bounds__(kThreads) void skinny_bf16_kernel(SkinnyArgs a) {
    __shared__ __attribute__((aligned(16))) float red[4][kSkinnyMaxM][kSkinnyCols];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int64_t cb = blockIdx.x;
    const int kb = blockIdx.y;
    const int64_t K = a.K, Ncol = a.Ncol;
    const int64_t col = cb * kSkinnyCols + 8 * c;
    const int64_t kw = (int64_t)kb * a.kblock + (int64_t)wave * 32 * KSTEPS;

    // ---- issue every load of this lane first (out-of-range rows/columns read zeros)
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.A, a.M * K * 2);
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(blockIdx.z ? a.Wu : a.W, K * Ncol * 2);
    const uint32_t arow = (uint32_t)(c * K * 2);
    uint4 af[KSTEPS];
    uint4 wr[KSTEPS][8];
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        const int64_t k0 = kw + 32 * t + 8 * g;
        af[t] = bload16(ra, (c < a.M && k0 < K) ? arow + (uint32_t)(k0 * 2) : kOOB);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t n = k0 + i;
            // rows past K fall outside the resource and read zeros; columns past
            // Ncol read finite neighbours that only reach unstored columns
            wr[t][i] = bload16(rw, (uint32_t)((n * Ncol + col) * 2));
        }
    }

    floatx4_t acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < KSTEPS; ++t) {
        uint4 cv[8];
        transpose8x8(wr[t], cv);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma16x16x32(af[t], cv[j], acc[j]);
    }

    // acc[j][r] = partial out[m = 4g + r][col + j]; sum the four waves in order
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float* dst = &red[wave][4 * g + r][8 * c];
        *reinterpret_cast<float4*>(dst) = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
    }
    __syncthreads();
    const int m = tid >> 4;           // 16 rows x 16 threads, 8 columns each
    const int cl = (tid & 15) * 8;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        v[i] = ((red[0][m][cl + i] + red[1][m][cl + i]) + red[2][m][cl + i]) + red[3][m][cl + i];
    const int64_t gc = cb * kSkinnyCols + cl;
    const bool outok = (m < a.M) && (gc < Ncol);

    if (a.nkb > 1 || a.gated) {
        if (gc < Ncol) {
            float* mine = (blockIdx.z ? a.part_u : a.part) + ((int64_t)kb * kSkinnyMaxM + m) * Ncol + gc;
            *reinterpret_cast<float4*>(mine) = make_float4(v[0], v[1], v[2], v[3]);
            *reinterpret_cast<float4*>(mine + 4) = make_float4(v[4], v[5], v[6], v[7]);
        }
        return;
    }
    if (!outok) return;
    if (a.bias) {
        uint4 bb = ld16(a.bias + gc);
        uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] += bf16_lo(bw[i]);
            v[2 * i + 1] += bf16_hi(bw[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = apply_act(a.act, v[i]);
    uint4 o = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7]));
    *reinterpret_cast<uint4*>(a.out + (int64_t)m * Ncol + gc) = o;
}

// Sum of the K-block partials of 4 columns, K blocks in ascending order.
__device__ __forceinline__ void sum_kblocks(const float* src, int nkb, int64_t kstride,
                                            float (&y)[4]) {
    y[0] = y[1] = y[2] = y[3] = 0.f;
    for (int q0 = 0; q0 < nkb; q0 += 2 * kBatch) {
        float4 t[2 * kBatch];
#pragma unroll
        for (int j = 0; j < 2 * kBatch; ++j) {   // all loads of a batch in flight at once
            const int q = (q0 + j < nkb) ? q0 + j : q0;
            t[j] = *reinterpret_cast<const float4*>(src + q * kstride);
        }
#pragma unroll
        for (int j = 0; j < 2 * kBatch; ++j) {
            if (q0 + j < nkb) {
                y[0] += t[j].x; y[1] += t[j].y; y[2] += t[j].z; y[3] += t[j].w;
            }
        }
    }
}

// out[m][c] = act(sum_kb part[kb][m][c] + bias[c]), K blocks in ascending order;
// gated: out[m][c] = silu(sum_kb part[kb][m][c]) * sum_kb part_u[kb][m][c].
// One thread per 4 output columns; small blocks so the few thousand threads
// spread over many CUs (the partials are L2/MALL-resident, just written).
template <bool kGated>
__global__ __launch_bounds__(64) void skinny_reduce_kernel(const float* __restrict__ part,
                                                           const float* __restrict__ part_u,
                                                           int nkb,
                                                           const uint16_t* __restrict__ bias,
                                                           uint16_t* __restrict__ out, int64_t M,
                                                           int64_t Ncol, int act) {
    const int64_t nvec = M * (Ncol / 4);
    const int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (v >= nvec) return;
    const int64_t m = v / (Ncol / 4);
    const int64_t c = (v - m * (Ncol / 4)) * 4;
    const int64_t kstride = (int64_t)kSkinnyMaxM * Ncol;
    float y[4];
    sum_kblocks(part + m * Ncol + c, nkb, kstride, y);
    if constexpr (kGated) {
        float u[4];
        sum_kblocks(part_u + m * Ncol + c, nkb, kstride, u);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = silu(y[i]) * u[i];
        *reinterpret_cast<uint2*>(out + m * Ncol + c) =
            make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        return;
    }
    if (bias) {
        const uint2 bb = *reinterpret_cast<const uint2*>(bias + c);
        y[0] += bf16_lo(bb.x);
        y[1] += bf16_hi(bb.x);
        y[2] += bf16_lo(bb.y);
        y[3] += bf16_hi(bb.y);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = apply_act(act, y[i]);
    *reinterpret_cast<uint2*>(out + m * Ncol + c) =
        make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
}

constexpr int kKSteps = 2;   // 32-deep MFMA steps per wave (two measured best at M = 16: 18.8 us per FFN call against 20.3 with one and 23.1 with four)
constexpr int64_t kKBlock = 4 * 32 * kKSteps;

}  // namespace

int64_t skinny_kblock(int64_t, int64_t) { return kKBlock; }

size_t skinny_partial_floats(int64_t K, int64_t Ncol) {
    int64_t nkb = (K + kKBlock - 1) / kKBlock;
    return nkb > 1 ? (size_t)(nkb * kSkinnyMaxM * Ncol) : 0;
}

size_t skinny_gated_partial_floats(int64_t K, int64_t Ncol) {
    return (size_t)(((K + kKBlock - 1) / kKBlock) * kSkinnyMaxM * Ncol);
}


hipError_t launch_skinny_bf16(const uint16_t* A, const uint16_t* W, const uint16_t* bias,
                              uint16_t* out, float* part, int64_t M, int64_t K, int64_t Ncol,
                              int act, hipStream_t stream) {
    SkinnyArgs a;
    a.A = A;
    a.W = W;
    a.Wu = W;
    a.bias = bias;
    a.out = out;
    a.part = part;
    a.part_u = part;
    a.gated = 0;
    a.M = M;
    a.K = K;
    a.Ncol = Ncol;
    a.kblock = kKBlock;
    a.nkb = (int)((K + kKBlock - 1) / kKBlock);
    a.act = act;
    dim3 grid((unsigned)((Ncol + kSkinnyCols - 1) / kSkinnyCols), (unsigned)a.nkb);
    hipLaunchKernelGGL(skinny_bf16_kernel<kKSteps>, grid, dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.nkb <= 1) return e;
    const int64_t nvec = M * (Ncol / 4);
    hipLaunchKernelGGL(skinny_reduce_kernel<false>, dim3((unsigned)((nvec + 63) / 64)), dim3(64), 0,
                       stream, part, part, a.nkb, bias, out, M, Ncol, act);
    return hipGetLastError();
}

hipError_t launch_skinny_swiglu_bf16(const uint16_t* A, const uint16_t* Wg, const uint16_t* Wu,
                                     uint16_t* out, float* part_g, float* part_u, int64_t M,
                                     int64_t K, int64_t Ncol, hipStream_t stream) {
    SkinnyArgs a;
    a.A = A;
    a.W = Wg;
    a.Wu = Wu;
    a.bias = nullptr;
    a.out = out;
    a.part = part_g;
    a.part_u = part_u;
    a.M = M;
    a.K = K;
    a.Ncol = Ncol;
    a.kblock = kKBlock;
    a.nkb = (int)((K + kKBlock - 1) / kKBlock);
    a.act = 0;
    a.gated = 1;
    dim3 grid((unsigned)((Ncol + kSkinnyCols - 1) / kSkinnyCols), (unsigned)a.nkb, 2);
    hipLaunchKernelGGL(skinny_bf16_kernel<kKSteps>, grid, dim3(kThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nvec = M * (Ncol / 4);
    hipLaunchKernelGGL(skinny_reduce_kernel<true>, dim3((unsigned)((nvec + 63) / 64)), dim3(64), 0,
                       stream, part_g, part_u, a.nkb, nullptr, out, M, Ncol, 0);
    return hipGetLastError();
}

}  // namespace ffn
