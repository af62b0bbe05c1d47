// ffn_fused.hip -- the fused two-layer FFN for bf16 inputs, H kept in LDS.
//
// Method: the kernel-fusion / tensor-parallelism post (brunomaga.github.io),
// section "Step 1: fusing the two linear layers".  The first layer is tiled
// as usual; the bias and the activation are applied to each H tile alone; the
// finished H tile is multiplied by the matching rows of W2 (the block-product
// equation Y_ik = sum_j H_ij (W2)_jk) and the products are accumulated into Y.
// H never leaves the chip.
//
// gfx950 design (differs from the page's, which targets a GPU with
// asynchronous tile reductions into global memory):
//  * one workgroup = 64 token rows x one hidden chunk of C columns (C = 448
//    or 512).  GEMM1 (K = N) runs on bf16 MFMA with fp32 accumulators; the
//    epilogue adds b1, applies the activation, rounds once to bf16 and writes
//    the 64 x C tile of H into LDS in the operand layout GEMM2 reads;
//  * GEMM2 sweeps the output columns in passes of 512, reading H from LDS and
//    streaming W2; each pass stores an fp32 partial of Y for this hidden chunk
//    (split-O).  A separate pass sums the chunks in ascending order, adds b2
//    once (the tensor-parallel equation: the bias is added after the sum) and
//    casts.  No floating-point atomics: results are bitwise reproducible.
//  * weights are row-major (N x O, O x P: output index contiguous).  The MFMA
//    wants k-contiguous operands, so each thread loads an 8x8 block (8 rows of
//    16 bytes), transposes it in registers and writes 8 k-contiguous chunks to
//    the swizzled LDS tile.
//  * the grouped form (Mixture-of-Experts) takes its rows from a tile table:
//    expert id, first row of the expert's sorted token list, valid rows; X
//    rows are gathered by token id on load.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;
constexpr int kXStage = kBM * kBK * 2;  // bytes of one X k-slab in LDS
constexpr int kW2Stage = kBN2 * kBK * 2;

template <int C>
struct FusedCfg {
    static constexpr int kFO = C / 64;               // 16-wide hidden fragments per wave
    static constexpr int kW1Stage = C * kBK * 2;
    static constexpr int kStage1 = kXStage + kW1Stage;
    static constexpr int kStageBytes = (kStage1 > kW2Stage) ? kStage1 : kW2Stage;
    static constexpr int kHOff = 2 * kStageBytes;
    static constexpr int kHSlab = kBM * kBK * 2;     // one 32-deep slab of H
    static constexpr int kLds = kHOff + (C / kBK) * kHSlab;
    static constexpr int kW1Threads = (C / 8) * 4;   // threads owning an 8x8 W1 block
    static_assert(C % 64 == 0, "chunk must split evenly over four waves");
    static_assert(kW1Threads <= kThreads, "one W1 block per thread at most");
};

struct FusedArgs {
    const uint16_t* X;
    const uint16_t* W1;
    const uint16_t* b1;
    const uint16_t* W2;
    float* part;
    int64_t M, N, O, P;
    int64_t rows_out;     // rows of each split in `part`
    int64_t row_blocks;   // row tiles used for the unit mapping
    int splits;
    int act1;
    GroupedRows g;
};

// Unit -> (row tile, hidden chunk).  Workgroups are dispatched round-robin
// over the 8 XCDs; when the row tiles divide evenly, all chunks of one row
// tile are given to the same XCD so they share its L2 (the X rows) and run
// at the same time.
__device__ __forceinline__ void map_unit(int64_t unit, int64_t row_blocks, int splits,
                                         int64_t* rb, int* s) {
    if ((row_blocks & 7) == 0) {
        int64_t xcd = unit & 7;
        int64_t j = unit >> 3;
        *rb = (j / splits) * 8 + xcd;
        *s = (int)(j % splits);
    } else {
        *rb = unit / splits;
        *s = (int)(unit % splits);
    }
}

template <int C, bool kGrouped>
__global__ __launch_bounds__(kThreads, 1) void fused_ffn_bf16_kernel(FusedArgs a) {
    using Cfg = FusedCfg<C>;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;   // fragment index
    const int lg = lane >> 4;   // fragment k-group

    int64_t rb;
    int s;
    map_unit(blockIdx.x, a.row_blocks, a.splits, &rb, &s);

    // ---- rows of this tile
    int64_t row0;
    int valid;
    int64_t expert = 0;
    if constexpr (kGrouped) {
        if (rb >= (int64_t)(*a.g.tile_count)) return;
        const int32_t* t = a.g.tiles + rb * 3;
        expert = t[0];
        row0 = t[1];
        valid = t[2];
    } else {
        row0 = rb * kBM;
        if (row0 >= a.M) return;
        valid = (int)((a.M - row0) < kBM ? (a.M - row0) : kBM);
    }
    const int64_t N = a.N, O = a.O, P = a.P;
    const uint16_t* W1 = a.W1 + expert * a.g.w1_stride;
    const uint16_t* W2 = a.W2 + expert * a.g.w2_stride;
    const uint16_t* b1 = a.b1 ? a.b1 + expert * a.g.b1_stride : nullptr;
    const int64_t o0 = (int64_t)s * C;
    const int64_t oc = (O - o0) < C ? (O - o0) : C;  // valid hidden columns of this chunk

    // ---- per-thread load roles
    // X slab: thread -> (row xr, k-group xg); 16 consecutive threads share xg.
    const int xr = (tid & 15) + 16 * (tid >> 6);
    const int xg = (tid >> 4) & 3;
    const uint16_t* xrow = nullptr;
    if (xr < valid) {
        int64_t token;
        if constexpr (kGrouped) token = a.g.sorted[row0 + xr] / a.g.k;
        else token = row0 + xr;
        xrow = a.X + token * N;
    }
    // weight blocks: thread -> (k-group wg, 8-column group wc)
    const int wg = tid & 3;
    const int wc = tid >> 2;
    const bool w1_role = tid < Cfg::kW1Threads;
    const bool w1_colok = w1_role && (8 * wc < oc);
    const uint16_t* w1col = W1 + o0 + 8 * wc;

    char* const hreg = smem + Cfg::kHOff;

    // =========================== GEMM1: A^T = W1_chunk^T X^T ===============
    uint4 xv;
    uint4 wv[8];
    auto load1 = [&](int64_t k0) {
        int64_t kx = k0 + 8 * xg;
        xv = (xrow && kx < N) ? ld16(xrow + kx) : zero16();
        if (w1_role) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int64_t n = k0 + 8 * wg + i;
                wv[i] = (w1_colok && n < N) ? ld16(w1col + n * O) : zero16();
            }
        }
    };
    auto store1 = [&](int buf) {
        char* sx = smem + buf * Cfg::kStageBytes;
        char* sw = sx + kXStage;
        *reinterpret_cast<uint4*>(sx + frag_off(xr, xg)) = xv;
        if (w1_role) {
            uint4 cv[8];
            transpose8x8(wv, cv);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint4*>(sw + frag_off(8 * wc + j, wg)) = cv[j];
        }
    };

    floatx4_t acc[Cfg::kFO][4];
#pragma unroll
    for (int i = 0; i < Cfg::kFO; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const int64_t nk = (N + kBK - 1) / kBK;
    load1(0);
    store1(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
        const int cur = (int)(kt & 1);
        if (kt + 1 < nk) load1((kt + 1) * kBK);
        const char* sx = smem + cur * Cfg::kStageBytes;
        const char* sw = sx + kXStage;
        uint4 bx[4];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) bx[fm] = ld16(sx + frag_off(16 * fm + li, lg));
#pragma unroll
        for (int fo = 0; fo < Cfg::kFO; ++fo) {
            uint4 aw = ld16(sw + frag_off(16 * (wave * Cfg::kFO + fo) + li, lg));
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) acc[fo][fm] = mfma16x16x32(aw, bx[fm], acc[fo][fm]);
        }
        if (kt + 1 < nk) store1(cur ^ 1);
        __syncthreads();
    }

    // =========================== GEMM2 setup ==============================
    const int64_t np = (P + kBN2 - 1) / kBN2;
    const int nk2 = (int)((oc + kBK - 1) / kBK);
    const int64_t nsteps = np * nk2;
    const uint16_t* w2base = W2 + (o0 + 8 * wg) * P + 8 * wc;

    auto load2 = [&](int64_t step) {
        int64_t pt = step / nk2;
        int ks = (int)(step - pt * nk2);
        int64_t p = pt * kBN2 + 8 * wc;
        int64_t orow = (int64_t)ks * kBK;   // relative to o0 + 8*wg
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            int64_t o = orow + 8 * wg + i;  // relative to o0
            wv[i] = (o < oc && p < P) ? ld16(w2base + (orow + i) * P + pt * kBN2) : zero16();
        }
    };
    auto store2 = [&](int buf) {
        char* sw = smem + buf * Cfg::kStageBytes;
        uint4 cv[8];
        transpose8x8(wv, cv);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint4*>(sw + frag_off(8 * wc + j, wg)) = cv[j];
    };

    if (nsteps > 0) load2(0);

    // ---- epilogue 1: H = act(A + b1) -> bf16 -> LDS (GEMM2 operand layout)
#pragma unroll
    for (int fo = 0; fo < Cfg::kFO; ++fo) {
        const int ol = 16 * (wave * Cfg::kFO + fo) + 4 * lg;  // first of 4 hidden cols
        const int64_t og = o0 + ol;
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        const bool colok = og < O;  // O % 8 == 0, so the 4 columns are all in or all out
        if (colok && b1) {
            uint2 bb = *reinterpret_cast<const uint2*>(b1 + og);
            bias[0] = bf16_lo(bb.x);
            bias[1] = bf16_hi(bb.x);
            bias[2] = bf16_lo(bb.y);
            bias[3] = bf16_hi(bb.y);
        }
        const int slab = ol / kBK;
        const int g = (ol % kBK) / 8;
        const int e = ol % 8;
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) {
            float h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[r] = colok ? apply_act(a.act1, acc[fo][fm][r] + bias[r]) : 0.f;
            uint2 pk = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            *reinterpret_cast<uint2*>(hreg + slab * Cfg::kHSlab + frag_off(16 * fm + li, g) +
                                      2 * e) = pk;
        }
    }

    // =========================== GEMM2: Ypart^T = W2_chunk^T H^T ==========
    floatx4_t acc2[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc2[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    if (nsteps > 0) store2(0);
    __syncthreads();
    float* const part = a.part + (int64_t)s * a.rows_out * P;
    for (int64_t step = 0; step < nsteps; ++step) {
        const int cur = (int)(step & 1);
        const int64_t pt = step / nk2;
        const int ks = (int)(step - pt * nk2);
        if (step + 1 < nsteps) load2(step + 1);
        const char* sw = smem + cur * Cfg::kStageBytes;
        const char* hs = hreg + ks * Cfg::kHSlab;
        uint4 bh[4];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) bh[fm] = ld16(hs + frag_off(16 * fm + li, lg));
#pragma unroll
        for (int fp = 0; fp < 8; ++fp) {
            uint4 aw = ld16(sw + frag_off(128 * wave + 16 * fp + li, lg));
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) acc2[fp][fm] = mfma16x16x32(aw, bh[fm], acc2[fp][fm]);
        }
        if (ks == nk2 - 1) {
            // store this pass's partial: lane holds 4 consecutive columns of row m
#pragma unroll
            for (int fp = 0; fp < 8; ++fp) {
                const int64_t p = pt * kBN2 + 128 * wave + 16 * fp + 4 * lg;
#pragma unroll
                for (int fm = 0; fm < 4; ++fm) {
                    const int m = 16 * fm + li;
                    if (m < valid && p < P) {
                        float4 v = make_float4(acc2[fp][fm][0], acc2[fp][fm][1], acc2[fp][fm][2],
                                               acc2[fp][fm][3]);
                        *reinterpret_cast<float4*>(part + (row0 + m) * P + p) = v;
                    }
                    acc2[fp][fm] = floatx4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
        if (step + 1 < nsteps) store2(cur ^ 1);
        __syncthreads();
    }
}

// ---------------------------------------------------------------- reduce

template <bool kYF32, bool kBF32>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const float* __restrict__ part,
                                                            int splits, const void* b2,
                                                            void* Y, int64_t M, int64_t P,
                                                            int act2) {
    const int64_t nvec = M * (P / 8);
    const int64_t split_stride = M * P;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = v / (P / 8);
        const int64_t p = (v - m * (P / 8)) * 8;
        const float* src = part + m * P + p;
        float4 lo = *reinterpret_cast<const float4*>(src);
        float4 hi = *reinterpret_cast<const float4*>(src + 4);
        for (int s = 1; s < splits; ++s) {
            const float* q = src + s * split_stride;
            float4 a = *reinterpret_cast<const float4*>(q);
            float4 b = *reinterpret_cast<const float4*>(q + 4);
            lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
            hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
        }
        float y[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (b2) {
            if constexpr (kBF32) {
                const float* bb = reinterpret_cast<const float*>(b2) + p;
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] += bb[i];
            } else {
                uint4 bb = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(b2) + p);
                uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y[2 * i] += bf16_lo(bw[i]);
                    y[2 * i + 1] += bf16_hi(bw[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) y[i] = apply_act(act2, y[i]);
        if constexpr (kYF32) {
            float* dst = reinterpret_cast<float*>(Y) + m * P + p;
            *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(y[4], y[5], y[6], y[7]);
        } else {
            uint4 o = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                 pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(Y) + m * P + p) = o;
        }
    }
}

template <int C, bool G>
hipError_t launch_fused_impl(const FusedArgs& a, int64_t units, hipStream_t stream) {
    using Cfg = FusedCfg<C>;
    auto kern = fused_ffn_bf16_kernel<C, G>;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::kLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(kThreads), Cfg::kLds, stream, a);
    return hipGetLastError();
}

}  // namespace

int fused_pick_chunk(int64_t O) {
    // prefer the chunk that divides O exactly with the fewest splits
    if (O % 512 == 0) return 512;
    if (O % 448 == 0) return 448;
    return 512;
}

int fused_num_splits(int64_t O, int chunk) { return (int)((O + chunk - 1) / chunk); }

hipError_t launch_fused_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* b1,
                             const uint16_t* W2, float* part, int64_t M, int64_t N, int64_t O,
                             int64_t P, int act1, int chunk, int64_t row_blocks,
                             int64_t rows_out, const GroupedRows* grouped, hipStream_t stream) {
    FusedArgs a;
    a.X = X;
    a.W1 = W1;
    a.b1 = b1;
    a.W2 = W2;
    a.part = part;
    a.M = M;
    a.N = N;
    a.O = O;
    a.P = P;
    a.rows_out = rows_out;
    a.row_blocks = row_blocks;
    a.splits = fused_num_splits(O, chunk);
    a.act1 = act1;
    if (grouped) a.g = *grouped;
    const int64_t units = row_blocks * a.splits;
    if (units <= 0) return hipSuccess;
    if (chunk == 448)
        return grouped ? launch_fused_impl<448, true>(a, units, stream)
                       : launch_fused_impl<448, false>(a, units, stream);
    return grouped ? launch_fused_impl<512, true>(a, units, stream)
                   : launch_fused_impl<512, false>(a, units, stream);
}

hipError_t launch_reduce_splits(const float* part, int splits, const void* b2, int b2_f32,
                                void* Y, int y_f32, int64_t M, int64_t P, int act2,
                                hipStream_t stream) {
    const int64_t nvec = M * (P / 8);
    if (nvec <= 0) return hipSuccess;
    int64_t blocks = (nvec + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    dim3 g((unsigned)blocks), b(256);
    if (y_f32) {
        if (b2_f32) hipLaunchKernelGGL((reduce_splits_kernel<true, true>), g, b, 0, stream, part, splits, b2, Y, M, P, act2);
        else hipLaunchKernelGGL((reduce_splits_kernel<true, false>), g, b, 0, stream, part, splits, b2, Y, M, P, act2);
    } else {
        if (b2_f32) hipLaunchKernelGGL((reduce_splits_kernel<false, true>), g, b, 0, stream, part, splits, b2, Y, M, P, act2);
        else hipLaunchKernelGGL((reduce_splits_kernel<false, false>), g, b, 0, stream, part, splits, b2, Y, M, P, act2);
    }
    return hipGetLastError();
}

}  // namespace ffn
