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
constexpr int kBK = 32;                // k-stage depth of both products (one MFMA k-step)
constexpr int kFrag = 1024;            // bytes of one 16-index x 32-deep operand fragment
constexpr int kSub = kBM * kBK * 2;    // one 32-deep slab of X or H in LDS: 4 KiB

// LDS layout of a row-major weight stage (32 k-rows x `cols` columns), filled by
// direct global->LDS loads and read back through the transposing LDS read.
// The stage is cut into 1 KiB blocks of 8 k-rows x 64 columns, block
// (r, c) at (r * cols/64 + c) KiB.  Inside a block the 16-byte unit holding
// row kk (0..7) and 8-column group u (0..7) sits at slot 8u + (kk ^ 4(u&1)):
// the loading lane l writes slot l, and the 16 lanes of one transposing read
// (4 rows x 2 neighbouring 8-column groups) hit 8 distinct 16-byte slots of a
// 128-byte window -- no bank conflicts on either side.
__device__ __forceinline__ uint32_t wtile_dma_row(int l) { return (l & 7) ^ (((l >> 3) & 1) << 2); }

// Byte offset, inside a weight stage with `nb` 64-column blocks per row group,
// of the 8-byte chunk that lane l of a transposing read supplies for operand
// fragment f (columns 16f..16f+15), half t (k-rows 8g+4t..8g+4t+3).
__device__ __forceinline__ uint32_t wtile_tr_off(int l, int nb, int f, int t) {
    const int g = l >> 4, s = l & 15, j = s >> 2, q = s & 3;
    const int c8 = 2 * f + (q >> 1);
    const int slot = 8 * (c8 & 7) + ((j + 4 * t) ^ ((c8 & 1) << 2));
    return (uint32_t)((g * nb + (c8 >> 3)) * kFrag + 16 * slot + 8 * (q & 1));
}

template <int C>
struct FusedCfg {
    static constexpr int kFO = C / 64;                 // hidden fragments per wave
    static constexpr int kNB1 = C / 64;                // W1 stage: 64-column blocks per row group
    static constexpr int kNB2 = kBN2 / 64;             // W2 stage: 8
    static constexpr int kKS = C / kBK;                // GEMM2 k-stages per output pass
    static constexpr int kW1Stage = 4 * kNB1 * kFrag;  // 32 x C bf16
    static constexpr int kStage1 = kSub + kW1Stage;    // X slab + W1 slab
    static constexpr int kStage2 = 4 * kNB2 * kFrag;   // 32 x 512 bf16 = 32 KiB
    static constexpr int kHBytes = kKS * kSub;         // H: C/32 slabs of 64 x 32
    static constexpr int kNS1 = 4;                     // GEMM1 stages in flight
    static constexpr int kNS2 = (kHBytes + 3 * kStage2 <= 152 * 1024) ? 3 : 2;
    static constexpr int kD1 = 1 + kNB1;               // DMA instructions per wave per GEMM1 stage
    static constexpr int kD2 = kNB2;                   // ... per GEMM2 stage
    static constexpr int kLds1 = kNS1 * kStage1;
    static constexpr int kLds2 = kHBytes + kNS2 * kStage2;
    static constexpr int kLds = kLds1 > kLds2 ? kLds1 : kLds2;
    static_assert(C % 64 == 0 && (4 * kNB1) % 4 == 0, "chunk must split over four waves");
    static_assert(kLds <= 160 * 1024, "LDS budget");
    static_assert(kNB1 <= kFO && kNB2 == 8, "one load slot per fragment");
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
// over the 8 XCDs (unit u runs on XCD u % 8), and each XCD has its own L2.
// When the split count divides 8 and the row tiles divide evenly, every XCD
// works on ONE hidden chunk (XCD x takes chunk x % splits and every
// (8/splits)-th row tile): its 32 workgroups then stream the same W1 and W2
// chunk in step, so each weight byte leaves HBM/MALL once per XCD group
// instead of once per XCD for every chunk.  Otherwise units are numbered
// row-major.
__device__ __forceinline__ void map_unit(int64_t unit, int64_t row_blocks, int splits,
                                         int64_t* rb, int* s) {
    const int g = (splits > 0 && 8 % splits == 0) ? 8 / splits : 0;
    if (g > 0 && row_blocks % g == 0) {
        const int x = (int)(unit & 7);
        const int64_t j = unit >> 3;
        *s = x % splits;
        *rb = (int64_t)(x / splits) + (int64_t)g * j;
    } else {
        *rb = unit / splits;
        *s = (int)(unit % splits);
    }
}

// Both products run the same pipeline: a ring of LDS stages filled by direct
// global->LDS loads issued NS-1 stages ahead.  At the top of every iteration
// each wave waits until its loads of the current stage have landed (the
// newer stages stay in flight), a barrier publishes the stage to all waves,
// the buffer freed by the previous stage is refilled, and the stage is
// multiplied out.  Loads past the end read zeros through out-of-range
// offsets, so every stage issues the same number of loads.
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

    // ---- X slab loads: wave w fills fragment w (rows 16w..16w+15); lane l
    // brings row 16w + l%16, k-group l/16, straight into fragment slot l.
    const int xr = 16 * wave + li;
    int32x4_t rx;
    uint32_t xrow_off = kOOB;
    if constexpr (kGrouped) {
        rx = make_srd(a.X, a.M * N * 2);
        if (xr < valid) xrow_off = (uint32_t)((a.g.sorted[row0 + xr] / a.g.k) * N * 2);
    } else {
        rx = make_srd(a.X + row0 * N, (int64_t)valid * N * 2);
        if (xr < valid) xrow_off = (uint32_t)(xr * N * 2);
    }
    // ---- weight loads: lane l brings k-row wtile_dma_row(l), column group l/8.
    // The W1 resource ends at the end of W1, so rows past N read zeros; columns
    // past this chunk's valid width read finite neighbours whose H columns the
    // epilogue forces to zero.
    const int32x4_t rw1 = make_srd(W1 + o0, (N * O - o0) * 2);
    const uint32_t w1_lane = (uint32_t)wtile_dma_row(lane) * (uint32_t)(O * 2) + 16u * (lane >> 3);

    // one W1 block (8 k-rows x 64 columns) of stage kt, block index blk
    auto dma_w1 = [&](int64_t kt, int buf, int blk) {
        char* sw = smem + buf * Cfg::kStage1 + kSub;
        const int r = blk / Cfg::kNB1, c = blk % Cfg::kNB1;
        const uint32_t base = (uint32_t)(((kt * kBK + 8 * r) * O + 64 * c) * 2);
        dma16(rw1, base + w1_lane, sw + blk * kFrag);
    };
    auto dma_x = [&](int64_t kt, int buf) {
        const int64_t kx = kt * kBK + 8 * lg;
        dma16(rx, kx < N ? xrow_off + (uint32_t)(kx * 2) : kOOB, smem + buf * Cfg::kStage1 + wave * kFrag);
    };
    auto issue1 = [&](int64_t kt, int buf) {
        dma_x(kt, buf);
#pragma unroll
        for (int i = 0; i < Cfg::kNB1; ++i) dma_w1(kt, buf, wave + 4 * i);
    };

    floatx4_t acc[Cfg::kFO][4];
#pragma unroll
    for (int i = 0; i < Cfg::kFO; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t trw1_0 = wtile_tr_off(lane, Cfg::kNB1, wave * Cfg::kFO, 0);
    const uint32_t trw1_1 = wtile_tr_off(lane, Cfg::kNB1, wave * Cfg::kFO, 1);
    // Multiply stage `buf` out of LDS while issuing the loads of stage kt_next
    // into buffer `nbuf`: one load after each fragment's four MFMAs, so that a
    // load waiting for the address unit never holds back a long run of MFMAs.
    auto step1 = [&](int buf, int64_t kt_next, int nbuf) {
        const char* st = smem + buf * Cfg::kStage1;
        const char* sw = st + kSub;
        uint4 bx[4], aw[Cfg::kFO];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) bx[fm] = ld16(st + fm * kFrag + 16 * lane);
#pragma unroll
        for (int fo = 0; fo < Cfg::kFO; ++fo) {
            // fragment offsets are linear in f: 256 bytes per 16 columns
            const uint2 lo = lds_read_tr16(sw + trw1_0 + 256 * fo);
            const uint2 hi = lds_read_tr16(sw + trw1_1 + 256 * fo);
            aw[fo] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
#pragma unroll
        for (int fo = 0; fo < Cfg::kFO; ++fo) {
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) acc[fo][fm] = mfma16x16x32(aw[fo], bx[fm], acc[fo][fm]);
            __builtin_amdgcn_sched_barrier(0);
            if (fo < Cfg::kNB1) dma_w1(kt_next, nbuf, wave + 4 * fo);
            __builtin_amdgcn_sched_barrier(0);
        }
        dma_x(kt_next, nbuf);
    };

    // =========================== GEMM1: A^T = W1_chunk^T X^T ===============
    const int64_t nk = (N + kBK - 1) / kBK;
#pragma unroll
    for (int i = 0; i < Cfg::kNS1 - 1; ++i) issue1(i, i);
    int cbuf = 0, ibuf = Cfg::kNS1 - 1;
    for (int64_t kt = 0; kt < nk; ++kt) {
        wait_vmcnt<Cfg::kD1 * (Cfg::kNS1 - 2)>();
        __syncthreads();
        step1(cbuf, kt + Cfg::kNS1 - 1, ibuf);
        cbuf = (cbuf + 1 == Cfg::kNS1) ? 0 : cbuf + 1;
        ibuf = (ibuf + 1 == Cfg::kNS1) ? 0 : ibuf + 1;
    }
    wait_vmcnt<0>();   // the stages loaded past the end still write LDS
    __syncthreads();

    // =========================== GEMM2 setup ==============================
    // W2 stage: 32 hidden rows x 512 output columns.  The W2 resource covers
    // exactly this chunk's rows, so rows past the chunk read zeros; columns
    // past P read finite neighbours that reach only unstored partial columns.
    const int32x4_t rw2 = make_srd(W2 + o0 * P, oc * P * 2);
    const uint32_t w2_lane = (uint32_t)wtile_dma_row(lane) * (uint32_t)(P * 2) + 16u * (lane >> 3);
    const int64_t np = (P + kBN2 - 1) / kBN2;
    char* const w2reg = smem + Cfg::kHBytes;
    auto dma_w2 = [&](int64_t step, int blk) {
        const int64_t pt = step / Cfg::kKS;
        const int ks = (int)(step - pt * Cfg::kKS);
        char* st = w2reg + (int)(step % Cfg::kNS2) * Cfg::kStage2;
        const int r = blk / Cfg::kNB2, c = blk % Cfg::kNB2;
        const uint32_t base = (uint32_t)(((int64_t)(ks * kBK + 8 * r) * P + pt * kBN2 + 64 * c) * 2);
        dma16(rw2, base + w2_lane, st + blk * kFrag);
    };
    auto issue2 = [&](int64_t step) {
#pragma unroll
        for (int i = 0; i < Cfg::kNB2; ++i) dma_w2(step, wave + 4 * i);
    };
    // the first W2 stages do not depend on H: start them before the epilogue
#pragma unroll
    for (int i = 0; i < Cfg::kNS2 - 1; ++i) issue2(i);

    // ---- epilogue 1: H = act(A + b1) -> bf16 -> LDS (GEMM2 operand layout)
    char* const hreg = smem;
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
        const int slab = ol / 32;
        const int g = (ol % 32) / 8;
        const int e = ol % 8;
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) {
            float h[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                h[r] = colok ? apply_act(a.act1, acc[fo][fm][r] + bias[r]) : 0.f;
            uint2 pk = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            *reinterpret_cast<uint2*>(hreg + slab * kSub + frag_off(16 * fm + li, g) + 2 * e) = pk;
        }
    }

    // =========================== GEMM2: Ypart^T = W2_chunk^T H^T ==========
    floatx4_t acc2[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc2[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    const uint32_t trw2_0 = wtile_tr_off(lane, Cfg::kNB2, 8 * wave, 0);
    const uint32_t trw2_1 = wtile_tr_off(lane, Cfg::kNB2, 8 * wave, 1);
    float* const part = a.part + (int64_t)s * a.rows_out * P;
    int64_t step = 0;   // global stage counter; the load ring runs across passes
    for (int64_t pt = 0; pt < np; ++pt) {
#pragma unroll 2
        for (int ks = 0; ks < Cfg::kKS; ++ks, ++step) {
            wait_vmcnt<Cfg::kD2 * (Cfg::kNS2 - 2)>();
            __syncthreads();
            const char* sw = w2reg + (int)(step % Cfg::kNS2) * Cfg::kStage2;
            const char* hs = hreg + ks * kSub;
            uint4 bh[4], aw[8];
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) bh[fm] = ld16(hs + frag_off(16 * fm + li, lg));
#pragma unroll
            for (int fp = 0; fp < 8; ++fp) {
                const uint2 lo = lds_read_tr16(sw + trw2_0 + 256 * fp);
                const uint2 hi = lds_read_tr16(sw + trw2_1 + 256 * fp);
                aw[fp] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            }
#pragma unroll
            for (int fp = 0; fp < 8; ++fp) {
#pragma unroll
                for (int fm = 0; fm < 4; ++fm)
                    acc2[fp][fm] = mfma16x16x32(aw[fp], bh[fm], acc2[fp][fm]);
                __builtin_amdgcn_sched_barrier(0);
                dma_w2(step + Cfg::kNS2 - 1, wave + 4 * fp);  // kNB2 == 8 loads per stage
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // this pass's partial: lane holds 4 consecutive columns of row m
#pragma unroll
        for (int fp = 0; fp < 8; ++fp) {
            const int64_t p = pt * kBN2 + 128 * wave + 16 * fp + 4 * lg;
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) {
                const int m = 16 * fm + li;
                if (m < valid && p < P) {
                    // streaming store: the partial is read once, by the reduction pass
                    floatx4_t* dst = reinterpret_cast<floatx4_t*>(part + (row0 + m) * P + p);
                    __builtin_nontemporal_store(acc2[fp][fm], dst);
                }
                acc2[fp][fm] = floatx4_t{0.f, 0.f, 0.f, 0.f};
            }
        }
    }
    wait_vmcnt<0>();   // no load into LDS may outlive the workgroup
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
