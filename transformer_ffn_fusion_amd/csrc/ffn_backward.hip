// ffn_backward.hip -- gradients of the two-layer FFN (act2 none) on MFMA.
//
// The kernel-fusion / tensor-parallelism post (brunomaga.github.io) names a
// fused backward pass as its next step, for the activation memory it saves:
// the forward keeps no H.  Here H is recomputed instead of stored.  With
// a = X W1 + b1, h = act1(a), Y = h W2 + b2 and the output gradient dY:
//
//   1. a = X W1 + b1      epilogue: h = act1(a), g = act1'(a)    (M x O, bf16)
//   2. dh = dY W2^T       epilogue: da = dh * g                  (M x O, bf16)
//   3. dX = da W1^T                                              (M x N, bf16)
//   4. dW1 = X^T da                                              (N x O, fp32)
//   5. dW2 = h^T dY                                              (O x P, fp32)
//   6. db1 = sum_m da, db2 = sum_m dY: column sums in a fixed order    (fp32)
//
// One GEMM kernel serves all five products: C[i][j] = sum_k A(i,k) B(j,k) with
// each operand either k-contiguous (element (i,k) at i*ld + k: X, dY, W2, da,
// W1 read as rows) or k-strided (element (i,k) at k*ld + i: W1 in step 1, X,
// da, h, dY in steps 4-5).  A k-contiguous operand is staged in LDS as 16 x 32
// fragments (the X-slab layout of the forward kernel); a k-strided one row by
// row in 8 x 64 blocks and read back k-contiguous through the transposing LDS
// read -- the layouts, and the checks of them, are the forward kernel's.
// Output tiles of 256 x 256 (eight waves of 128 x 64) when they fill the chip,
// else 128 x 128 (four waves of 64 x 64, two workgroups per CU); a 4-stage LDS
// ring filled by direct global->LDS loads.  Every output element is one
// workgroup's sum over the whole K in a fixed order: no atomics, bitwise
// reproducible for a given shape and device.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kGK = 32;                   // k-stage depth (one MFMA k-step)

// Output tile TI x TJ, WI x WJ waves of (TI/WI) x (TJ/WJ) each.  A stage holds
// TI and TJ operand indices x 32 k (TI/16 + TJ/16 units of 1 KiB, spread over
// the waves).  Bigger tiles and bigger wave tiles cut the L2 -> LDS bytes and
// the LDS -> register bytes per MFMA.
template <int TI_, int TJ_, int WI_, int WJ_, int NS_ = 4>
struct GemmCfg {
    static constexpr int TI = TI_, TJ = TJ_, WI = WI_, WJ = WJ_;
    static constexpr int kGNS = NS_;                            // LDS ring stages
    static constexpr int kWaves = WI * WJ;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int FI = TI / WI / 16, FJ = TJ / WJ / 16;   // fragments per wave
    static constexpr int kOpA = TI * kGK * 2;
    static constexpr int kStage = kOpA + TJ * kGK * 2;
    static constexpr int kLds = kGNS * kStage;
    static_assert(kGNS >= 3, "the ring keeps one stage being read and one landing");
    static constexpr int kUnits = TI / 16 + TJ / 16;
    static constexpr int kLoads = kUnits / kWaves;              // direct loads per wave per stage
    static_assert(TI % 64 == 0 && TJ % 64 == 0, "k-strided operands stage 64-index blocks");
    static_assert(FI * 16 * WI == TI && FJ * 16 * WJ == TJ, "whole fragments per wave");
    static_assert(kUnits % kWaves == 0, "every wave issues the same loads");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_HG = 2, EPI_MULG = 3 };

struct GemmArgs {
    const uint16_t* A;   // operand of the output rows i
    const uint16_t* B;   // operand of the output columns j
    int64_t lda, ldb;
    int64_t I, J, K;
    void* C;             // output, I x J, leading dimension J
    uint16_t* C2;        // EPI_HG: g = act1'(a), bf16, I x J
    const uint16_t* bias;  // EPI_HG: b1 over j (bf16) or null
    const uint16_t* G;   // EPI_MULG: g, bf16, I x J
    int act;
    int compact;         // XCD-compact tile order (else row-major), see gemm_tile
};

// act1'(x): ReLU' (0 at the kink), GELU-tanh' = s + 2 x s (1 - s) u'(x) with
// s = sigmoid(2u) = 0.5 (1 + tanh u), u = sqrt(2/pi) (x + 0.044715 x^3),
// u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2); none: 1.
__device__ __forceinline__ float act_grad(int act, float x) {
    if (act == ACT_RELU) return x > 0.0f ? 1.0f : 0.0f;
    if (act == ACT_GELU_TANH) {
        const float k = 0.7978845608028654f;
        const float u = k * x * (1.0f + 0.044715f * x * x);
        const float s = __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * u));
        return s + 2.0f * x * s * (1.0f - s) * k * (1.0f + 3.0f * 0.044715f * x * x);
    }
    return 1.0f;
}

// One operand's loads of the k-stage starting at k0 into LDS at `dst`: unit q
// (0 .. T/16-1) of an operand with T indices per tile.  k-contiguous: unit q =
// fragment q (indices 16q..16q+15 x 32 k; lane l brings index 16q + l/4,
// k-group (l&3)^((l>>3)&3), which lands in slot l of the fragment).
// k-strided: unit q = block (r, c) = (q / nb, q % nb) of 8 k-rows x 64
// indices, nb = T/64 blocks per row group (lane l brings slot l, see
// wtile_dma_off); rows at or past K read zeros.
template <bool kOuter, int T>
__device__ __forceinline__ void gemm_issue(const int32x4_t& rs, int64_t ld, int64_t n_idx,
                                           int64_t K, int64_t i0, int64_t k0, int q, int lane,
                                           char* dst) {
    uint32_t off = kOOB;
    if constexpr (!kOuter) {
        const int64_t i = i0 + 16 * q + (lane >> 2);
        const int64_t k = k0 + 8 * ((lane & 3) ^ ((lane >> 3) & 3));
        if (i < n_idx && k < K) off = (uint32_t)((i * ld + k) * 2);
        dma16(rs, off, dst + q * kFrag);
    } else {
        constexpr int nb = T / 64;
        const int r = q / nb, c = q % nb;
        const int64_t k = k0 + 8 * r + (lane >> 3);
        if (k < K)
            off = (uint32_t)(((k0 + 8 * r) * ld + i0 + 64 * c) * 2) + wtile_dma_off(lane, (uint32_t)(ld * 2));
        dma16(rs, off, dst + q * kFrag);
    }
}

// Operand fragment f (indices 16f..16f+15) of a stage, for this lane.
template <bool kOuter, int T>
__device__ __forceinline__ uint4 gemm_frag(const char* st, int f, int lane) {
    if constexpr (!kOuter) {
        return ld16(st + f * kFrag + 16 * xfrag_slot(lane & 15, lane >> 4));
    } else {
        const char* p = st + wtile_tr_base(lane, T / 64, f & 3) + 1024 * (f >> 2);
        const uint2 lo = lds_read_tr16(p);
        const uint2 hi = lds_read_tr16(p + 512);
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
}

// Workgroup -> output tile.  Workgroups are dispatched round-robin over the 8
// XCDs (workgroup w runs on XCD w % 8) and each XCD has its own L2.  Compact
// order: XCD x takes the contiguous run [x T, (x + 1) T) of a grouped tile
// order (groups of kGroupRows tile rows, rows fastest within a group), a
// compact rectangle (8 x 7 of the 32 x 14 tiles of a 4096 x 1792 output) whose
// A and B panels its L2 shares.  Row-major order gives every XCD every tile
// row and two tile columns (343 MB of HBM reads for the first product's 47 MB
// of operands).  Measured at the prefill shard (us): da 92 -> 84 compact,
// the first product 94 -> 98 (its k-strided W1 panels are the ones the
// row-major order shares), the weight gradients and dX unchanged.  Returns
// false for the padding workgroups of the compact order.
constexpr int kGroupRows = 8;

__device__ __forceinline__ bool gemm_tile(const GemmArgs& a, int TI, int TJ, int64_t* ti,
                                          int64_t* tj) {
    const int64_t nI = (a.I + TI - 1) / TI, nJ = (a.J + TJ - 1) / TJ;
    const int64_t ntiles = nI * nJ;
    if (!a.compact) {
        if ((int64_t)blockIdx.x >= ntiles) return false;
        *ti = blockIdx.x / nJ;
        *tj = blockIdx.x % nJ;
        return true;
    }
    const int64_t per = (ntiles + 7) / 8;
    const int64_t t = (int64_t)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (t >= ntiles) return false;
    const int64_t r = t / (kGroupRows * nJ);                 // row group
    const int64_t rows = (nI - r * kGroupRows) < kGroupRows ? (nI - r * kGroupRows) : kGroupRows;
    const int64_t rem = t - r * kGroupRows * nJ;
    *tj = rem / rows;
    *ti = r * kGroupRows + rem % rows;
    return true;
}

template <class Cfg, bool kAOuter, bool kBOuter, int kEpi>
__global__ __launch_bounds__(Cfg::kThreads) void gemm_bf16_kernel(GemmArgs a) {
    constexpr int FI = Cfg::FI, FJ = Cfg::FJ;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave / Cfg::WJ, wj = wave % Cfg::WJ;
    const int li = lane & 15, lg = lane >> 4;
    int64_t ti, tj;
    if (!gemm_tile(a, Cfg::TI, Cfg::TJ, &ti, &tj)) return;
    const int64_t i0 = ti * Cfg::TI;
    const int64_t j0 = tj * Cfg::TJ;
    const int64_t K = a.K;
    const int64_t nk = (K + kGK - 1) / kGK;
    // the resources span whole operands (every offset below 2^31 bytes)
    const int32x4_t ra = make_srd(a.A, (kAOuter ? K * a.lda : a.I * a.lda) * 2);
    const int32x4_t rb = make_srd(a.B, (kBOuter ? K * a.ldb : a.J * a.ldb) * 2);

    // wave w issues units w, w + W, ... of the stage (A's units first, then B's)
    auto issue = [&](int64_t kt, int buf) {
        char* st = smem + buf * Cfg::kStage;
        const int64_t k0 = kt * kGK;
#pragma unroll
        for (int u = 0; u < Cfg::kLoads; ++u) {
            const int q = wave + Cfg::kWaves * u;
            if (q < Cfg::TI / 16)
                gemm_issue<kAOuter, Cfg::TI>(ra, a.lda, a.I, K, i0, k0, q, lane, st);
            else
                gemm_issue<kBOuter, Cfg::TJ>(rb, a.ldb, a.J, K, j0, k0, q - Cfg::TI / 16, lane,
                                             st + Cfg::kOpA);
        }
    };

    floatx4_t acc[FI][FJ];   // [i fragment][j fragment]
#pragma unroll
    for (int x = 0; x < FI; ++x)
#pragma unroll
        for (int y = 0; y < FJ; ++y) acc[x][y] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    constexpr int kGNS = Cfg::kGNS;
#pragma unroll
    for (int s = 0; s < kGNS - 1; ++s)
        if (s < nk) issue(s, s);
    for (int64_t kt = 0; kt < nk; ++kt) {
        // stages kt .. min(kt + NS - 2, nk - 1) are in flight; stage kt must land
        if (kt + kGNS - 2 < nk) wait_vmcnt<Cfg::kLoads * (kGNS - 2)>();
        else wait_vmcnt<0>();
        __syncthreads();   // stage kt is complete everywhere; stage kt - 1 is read
        if (kt + kGNS - 1 < nk) issue(kt + kGNS - 1, (int)((kt + kGNS - 1) % kGNS));
        const char* st = smem + (kt % kGNS) * Cfg::kStage;
        uint4 fa[FI], fb[FJ];
#pragma unroll
        for (int x = 0; x < FI; ++x) fa[x] = gemm_frag<kAOuter, Cfg::TI>(st, FI * wi + x, lane);
#pragma unroll
        for (int y = 0; y < FJ; ++y)
            fb[y] = gemm_frag<kBOuter, Cfg::TJ>(st + Cfg::kOpA, FJ * wj + y, lane);
        // B first: the lane then holds four consecutive output columns of a row
#pragma unroll
        for (int x = 0; x < FI; ++x)
#pragma unroll
            for (int y = 0; y < FJ; ++y) acc[x][y] = mfma16x16x32(fb[y], fa[x], acc[x][y]);
    }

    // lane (li, lg) holds C[i0 + 16 (FI wi + x) + li][j0 + 16 (FJ wj + y) + 4 lg + r]
#pragma unroll
    for (int x = 0; x < FI; ++x) {
        const int64_t i = i0 + 16 * (FI * wi + x) + li;
        if (i >= a.I) continue;
#pragma unroll
        for (int y = 0; y < FJ; ++y) {
            const int64_t j = j0 + 16 * (FJ * wj + y) + 4 * lg;
            if (j >= a.J) continue;   // J % 8 == 0: the 4 columns are all in or all out
            const int64_t o = i * a.J + j;
            float v[4] = {acc[x][y][0], acc[x][y][1], acc[x][y][2], acc[x][y][3]};
            if constexpr (kEpi == EPI_F32) {
                *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.C) + o) =
                    make_float4(v[0], v[1], v[2], v[3]);
            } else if constexpr (kEpi == EPI_BF16) {
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.C) + o) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            } else if constexpr (kEpi == EPI_HG) {
                if (a.bias) {
                    const uint2 bb = *reinterpret_cast<const uint2*>(a.bias + j);
                    v[0] += bf16_lo(bb.x); v[1] += bf16_hi(bb.x);
                    v[2] += bf16_lo(bb.y); v[3] += bf16_hi(bb.y);
                }
                float h[4], g[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    h[r] = apply_act(a.act, v[r]);
                    g[r] = act_grad(a.act, v[r]);
                }
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.C) + o) =
                    make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
                *reinterpret_cast<uint2*>(a.C2 + o) =
                    make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
            } else {   // EPI_MULG
                const uint2 gg = *reinterpret_cast<const uint2*>(a.G + o);
                v[0] *= bf16_lo(gg.x); v[1] *= bf16_hi(gg.x);
                v[2] *= bf16_lo(gg.y); v[3] *= bf16_hi(gg.y);
                *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.C) + o) =
                    make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            }
        }
    }
}

// Column sums of two bf16 matrices (the bias gradients: da, M x O, and dY,
// M x P) into fp32, in a fixed order and without atomics, in two launches.
// Pass 1: workgroup (column group, row chunk) -- 64 columns x kColChunks-th of
// the rows; thread (r, c) adds rows r, r + 32, ... of its chunk for the eight
// columns 8c .. 8c + 7 (16-byte loads, eight rows in flight), then thread r = 0
// of each column group adds the 32 row-lane sums in ascending r and writes
// the chunk's partial.  Pass 2: one thread per column adds the kColChunks
// partials in ascending chunk order.  (One workgroup per 64 columns over all
// rows measured 11 us per matrix; the chunks give the loads 8x the CUs.)
constexpr int kColLanes = 32;
constexpr int kColChunks = 8;

__global__ __launch_bounds__(256) void colsum_partial_kernel(const uint16_t* __restrict__ A,
                                                             int64_t SA, const uint16_t* __restrict__ B,
                                                             int64_t SB, int64_t R,
                                                             float* __restrict__ part) {
    __shared__ float s_part[kColLanes][64 + 1];
    const int tid = threadIdx.x;
    const int c = tid & 7, r = tid >> 3;
    const int64_t ga = (SA + 63) / 64;
    const bool first = (int64_t)blockIdx.x < ga;   // which matrix this column group reads
    const uint16_t* src = first ? A : B;
    const int64_t S = first ? SA : SB;
    const int64_t col0 = (first ? (int64_t)blockIdx.x : (int64_t)blockIdx.x - ga) * 64;
    const int64_t col = col0 + 8 * c;
    const int64_t rows = (R + kColChunks - 1) / kColChunks;
    const int64_t r0 = (int64_t)blockIdx.y * rows;
    const int64_t r1 = (r0 + rows) < R ? (r0 + rows) : R;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (col < S) {
        int64_t row = r0 + r;
        for (; row + 7 * kColLanes < r1; row += 8 * kColLanes) {
            uint4 v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] = ld16(src + (row + q * kColLanes) * S + col);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t w[4] = {v[q].x, v[q].y, v[q].z, v[q].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += bf16_lo(w[e]);
                    acc[2 * e + 1] += bf16_hi(w[e]);
                }
            }
        }
        for (; row < r1; row += kColLanes) {
            const uint4 v = ld16(src + row * S + col);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += bf16_lo(w[e]);
                acc[2 * e + 1] += bf16_hi(w[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s_part[r][8 * c + e] = acc[e];
    __syncthreads();
    if (tid < 64) {
        const int64_t oc = col0 + tid;
        float t = 0.f;
        for (int q = 0; q < kColLanes; ++q) t += s_part[q][tid];
        // partials: [chunk][SA + SB], the first matrix's columns first
        if (oc < S) part[(int64_t)blockIdx.y * (SA + SB) + (first ? 0 : SA) + oc] = t;
    }
}

__global__ __launch_bounds__(256) void colsum_finish_kernel(const float* __restrict__ part,
                                                            int64_t SA, int64_t SB,
                                                            float* __restrict__ outA,
                                                            float* __restrict__ outB) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= SA + SB) return;
    float v[kColChunks];
#pragma unroll
    for (int q = 0; q < kColChunks; ++q) v[q] = part[(int64_t)q * (SA + SB) + j];
    float t = 0.f;
#pragma unroll
    for (int q = 0; q < kColChunks; ++q) t += v[q];
    if (j < SA) {
        if (outA) outA[j] = t;
    } else if (outB) {
        outB[j - SA] = t;
    }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* p, int64_t n) {
    for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

template <class Cfg, bool kAOuter, bool kBOuter, int kEpi>
hipError_t launch_gemm_cfg(const GemmArgs& a, hipStream_t stream) {
    auto kern = gemm_bf16_kernel<Cfg, kAOuter, kBOuter, kEpi>;
    static std::atomic<bool> lds_set[kMaxDevices] = {};
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), Cfg::kLds, lds_set);
    if (e != hipSuccess) return e;
    const int64_t ntiles = ((a.I + Cfg::TI - 1) / Cfg::TI) * ((a.J + Cfg::TJ - 1) / Cfg::TJ);
    const int64_t grid = a.compact ? 8 * ((ntiles + 7) / 8) : ntiles;   // see gemm_tile
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::kThreads), Cfg::kLds, stream, a);
    return hipGetLastError();
}

// Tile choice, measured at the prefill shard (4096 x 4096 x 1792 x 4096, us per
// product): 256 x 256 with eight waves of 128 x 64 wins when its tiles fill
// the chip (dX, 4096 x 4096 outputs: 83 -> 62), but leaves it half idle on the
// 4096 x 1792 outputs (97 -> 143); there the 128 x 128 tile (two workgroups
// per CU) stays best: 256 x 128 or 128 x 256 tiles with four waves of 128 x 64
// (one wave per SIMD) measured 101-127, with eight waves of 64 x 64 88-101,
// a 5-stage ring for the 256 x 256 tile 69 on dX; four extra waves that only
// issue the loads (as in the fused forward kernel) beside eight multiplying
// waves of 64 x 64 on 256 x 128 or 128 x 256 tiles 103-189 (register caps
// of three waves per SIMD).
using GemmSmall = GemmCfg<128, 128, 2, 2>;   // four waves of 64 x 64
using GemmLarge = GemmCfg<256, 256, 2, 4>;   // eight waves of 128 x 64

template <bool kAOuter, bool kBOuter, int kEpi>
hipError_t launch_gemm(const GemmArgs& a, hipStream_t stream) {
    if (a.I <= 0 || a.J <= 0) return hipSuccess;
    const int64_t large_tiles = ((a.I + GemmLarge::TI - 1) / GemmLarge::TI) *
                                ((a.J + GemmLarge::TJ - 1) / GemmLarge::TJ);
    if (large_tiles >= device_cus())
        return launch_gemm_cfg<GemmLarge, kAOuter, kBOuter, kEpi>(a, stream);
    return launch_gemm_cfg<GemmSmall, kAOuter, kBOuter, kEpi>(a, stream);
}

GemmArgs gemm_args(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, int64_t I,
                   int64_t J, int64_t K, void* C) {
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.lda = lda;
    g.ldb = ldb;
    g.I = I;
    g.J = J;
    g.K = K;
    g.C = C;
    g.C2 = nullptr;
    g.bias = nullptr;
    g.G = nullptr;
    g.act = 0;
    g.compact = 1;
    return g;
}

}  // namespace

size_t colsum_partial_floats(int64_t O, int64_t P) { return (size_t)kColChunks * (O + P); }

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t stream) {
    if (!p || n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_ffn_backward(const BackwardIO& io, hipStream_t stream, void** events,
                               int n_events) {
    const int64_t M = io.M, N = io.N, O = io.O, P = io.P;
    hipError_t e;
    // events[s] (when given) is recorded before step s + 1; events[6] after the last
    auto mark = [&](int s) -> hipError_t {
        if (!events || s >= n_events) return hipSuccess;
        return hipEventRecord(reinterpret_cast<hipEvent_t>(events[s]), stream);
    };
    if ((e = mark(0)) != hipSuccess) return e;
    // 1. a = X W1 + b1 -> h, g       (i = token, j = hidden; K = N; W1 k-strided)
    GemmArgs g1 = gemm_args(io.X, N, io.W1, O, M, O, N, io.H);
    g1.C2 = io.Gr;
    g1.bias = io.b1;
    g1.act = io.act1;
    g1.compact = 0;   // row-major order measured faster for this product (see gemm_tile)
    if ((e = launch_gemm<false, true, EPI_HG>(g1, stream)) != hipSuccess) return e;
    if ((e = mark(1)) != hipSuccess) return e;
    // 2. dh = dY W2^T -> da = dh * g (i = token, j = hidden; K = P; W2 rows)
    GemmArgs g2 = gemm_args(io.dY, P, io.W2, P, M, O, P, io.dA);
    g2.G = io.Gr;
    if ((e = launch_gemm<false, false, EPI_MULG>(g2, stream)) != hipSuccess) return e;
    if ((e = mark(2)) != hipSuccess) return e;
    // 3. dX = da W1^T                 (i = token, j = input column; K = O; W1 rows)
    GemmArgs g3 = gemm_args(io.dA, O, io.W1, O, M, N, O, io.dX);
    if ((e = launch_gemm<false, false, EPI_BF16>(g3, stream)) != hipSuccess) return e;
    if ((e = mark(3)) != hipSuccess) return e;
    // 4. dW1 = X^T da                 (i = input column, j = hidden; K = M; both k-strided)
    GemmArgs g4 = gemm_args(io.X, N, io.dA, O, N, O, M, io.dW1);
    if ((e = launch_gemm<true, true, EPI_F32>(g4, stream)) != hipSuccess) return e;
    if ((e = mark(4)) != hipSuccess) return e;
    // 5. dW2 = h^T dY                 (i = hidden, j = output column; K = M)
    GemmArgs g5 = gemm_args(io.H, O, io.dY, P, O, P, M, io.dW2);
    if ((e = launch_gemm<true, true, EPI_F32>(g5, stream)) != hipSuccess) return e;
    if ((e = mark(5)) != hipSuccess) return e;
    // 6. bias gradients: column sums of da and dY (a matrix whose gradient is
    // not wanted is skipped: zero columns)
    if (io.db1 || io.db2) {
        const int64_t SA = io.db1 ? O : 0, SB = io.db2 ? P : 0;
        const int64_t groups = (SA + 63) / 64 + (SB + 63) / 64;
        hipLaunchKernelGGL(colsum_partial_kernel, dim3((unsigned)groups, kColChunks), dim3(256), 0,
                           stream, io.dA, SA, io.dY, SB, M, io.colpart);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(colsum_finish_kernel, dim3((unsigned)((SA + SB + 255) / 256)), dim3(256),
                           0, stream, io.colpart, SA, SB, io.db1, io.db2);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return mark(6);
}

}  // namespace ffn
