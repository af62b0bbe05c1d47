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
//  * one workgroup = 64 token rows x one hidden chunk of C columns (C = 256,
//    448 or 512).  GEMM1 (K = N) runs on bf16 MFMA with fp32 accumulators; the
//    epilogue adds b1, applies the activation, rounds once to bf16 and writes
//    the 64 x C tile of H into LDS in the operand layout GEMM2 reads;
//  * GEMM2 sweeps the output columns in passes of 512, reading H from LDS and
//    streaming W2; each pass stores a partial of Y for this hidden chunk
//    (fp32 sums cut to a 16-bit significand: three bytes each)
//    (split-O).  A separate pass sums the chunks in ascending order, adds b2
//    once (the tensor-parallel equation: the bias is added after the sum) and
//    casts.  No floating-point atomics: results are bitwise reproducible.
//  * weights are row-major (N x O, O x P: output index contiguous).  The MFMA
//    wants k-contiguous operands: weight stages go to LDS row by row through
//    direct global->LDS loads (coalesced, no registers involved) and come back
//    k-contiguous through the gfx950 transposing LDS read (ds_read_b64_tr_b16);
//  * each workgroup runs 4 loader waves (they only issue the direct-to-LDS
//    loads) beside 4 multiplier waves (LDS reads + MFMA), one of each per SIMD,
//    so that the address unit's back-pressure never stalls the matrix cores;
//  * the grouped form (Mixture-of-Experts) takes its rows from a tile table:
//    expert id, first row of the expert's sorted token list, valid rows; X
//    rows are gathered by token id on load;
//  * the gated form (SwiGLU: same post, section "Benchmarks": a third weight
//    matrix gates the activation, no biases) keeps the same pipeline.  Its
//    first product is C wide but covers C/2 hidden columns: the left half of
//    the W1 stage comes from the gate matrix Wg, the right half from the up
//    matrix Wu, so each multiplier wave holds the gate and the up value of
//    the same hidden columns and the epilogue writes silu(gate) * up to H.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kMulWaves = 4;              // waves that multiply (one per SIMD)
constexpr int kThreads = 128 * kMulWaves; // ... plus as many waves that only load
constexpr int kBK = 32;                // k-stage depth of both products (one MFMA k-step)
constexpr int kSub = kBM * kBK * 2;    // one 32-deep slab of X or H in LDS: 4 KiB

// One first-product pass: a stage of 32 k-rows of X (64 rows) and of CP
// columns of W1, held in an NS-deep LDS ring.
template <int CP, int NS = 4>
struct PassCfg {
    static constexpr int kNB1 = CP / 64;               // W1 stage: 64-column blocks per row group
    static constexpr int kFO = CP / 64;                // fragments per multiplier wave (every 4th)
    static constexpr int kW1Stage = 4 * kNB1 * kFrag;  // 32 x CP bf16
    static constexpr int kStage1 = kSub + kW1Stage;    // X slab + W1 slab
    static constexpr int kNS1 = NS;                    // stages in the LDS ring
    static constexpr int kD1 = 1 + kNB1;               // loads per loader wave per stage
    static constexpr int kLds1 = kNS1 * kStage1;
    static_assert(CP % 64 == 0, "a pass splits over four waves in 16-column fragments");
    static_assert(kNS1 >= 3, "the multipliers read one stage ahead; the loaders need one more");
};

// Kernel configuration: pass A of CA first-product columns and, when CB > 0,
// a second pass B of CB columns over the next hidden columns of the chunk.
// The gated form halves each pass into gate and up columns (hidden columns
// per pass = CP / 2).  H is kKS slabs of 64 x 32 at LDS offset kHOff: slabs
// 0 .. kSlabsB-1 hold pass B's hidden columns, the rest pass A's.  With two
// passes, pass B's ring ends where pass A's H begins (pass A's H must survive
// pass B) and pass B's own H goes into the top of its ring once the pass is
// over, so H is contiguous and the whole kernel needs max(ring A, ring B + H A).
// kHLo (compensated H): H is held as two bf16 tiles, hi = bf16(h) and
// lo = bf16(h - hi), kLoOff bytes apart; the second product multiplies both
// with the same W2 operand into the same fp32 accumulators, so the error H
// adds to Y is that of a ~16-bit significand instead of bf16's 8 bits.
template <int CA, int CB, bool kGated, bool kHLo = false>
struct FusedCfg {
    // the dense two-pass chunk (448 + 448 hidden columns) fits the LDS only
    // with a 3-deep ring for its second pass
    static constexpr int kNSB = (CB > 0 && !kGated) ? 3 : 4;
    // chunks of at most 256 columns (an expert's share of a sharded layer) run
    // half a chip of short units whose first product waits on memory latency:
    // a 6-deep ring keeps more of it in flight (expert-sharded MoE share:
    // 140 -> 133.5 us; 8 stages measured the same)
    using PA = PassCfg<CA, (CA <= 256 ? 6 : 4)>;
    using PB = PassCfg<(CB > 0 ? CB : 64), kNSB>;      // unused with one pass
    static constexpr bool kTwoPass = CB > 0;
    static constexpr int kHidA = kGated ? CA / 2 : CA;
    static constexpr int kHidB = kTwoPass ? (kGated ? CB / 2 : CB) : 0;
    static constexpr int kHid = kHidA + kHidB;         // hidden columns per chunk
    static constexpr int kKS = kHid / kBK;             // GEMM2 k-stages per output pass
    static constexpr int kSlabsB = kHidB / kBK;
    static constexpr int kHOff = kTwoPass ? PB::kLds1 - kSlabsB * kSub : 0;
    // compensated H: a second set of kKS slabs holds the bf16 rounding residue
    static constexpr int kLoOff = kKS * kSub;
    static constexpr int kHEnd = kHOff + (kHLo ? 2 : 1) * kKS * kSub;
    static constexpr int kLds = PA::kLds1 > kHEnd ? PA::kLds1 : kHEnd;
    // second product (P a multiple of 128): per-wave staging of packed
    // partials (8 rows x 384 bytes per wave), below H when H leaves room
    // there, else above it
    static constexpr int kStgBytes = 8 * 8 * 384;
    static constexpr int kStgOff = kHOff >= kStgBytes ? 0 : kHEnd;
    static constexpr int kLdsAll = kStgOff + kStgBytes > kLds ? kStgOff + kStgBytes : kLds;
    static_assert(kStgOff == 0 ? kStgBytes <= kHOff : true, "the staging area fits below H");
    static_assert(kLdsAll <= 160 * 1024, "LDS budget with the staging area");
    static_assert(kHidA % kBK == 0 && kHidB % kBK == 0, "passes cover whole H slabs");
    static_assert(!kGated || (PA::kNB1 % 2 == 0 && (!kTwoPass || PB::kNB1 % 2 == 0)),
                  "gate and up halves are whole 64-column blocks");
    static_assert(kKS % 2 == 0, "GEMM2 runs its stages in pairs");
    static_assert(kBN2 == 64 * 2 * kMulWaves, "each of the eight waves owns 64 columns of a pass");
    static_assert(kLds <= 160 * 1024, "LDS budget");
};

struct FusedArgs {
    const uint16_t* X;
    const uint16_t* W1;   // gated form: the gate matrix Wg
    const uint16_t* W1u;  // gated form: the up matrix Wu (unused otherwise)
    const uint16_t* b1;
    const uint16_t* W2;
    char* part;           // packed partials, kPartBytes each: [splits][rows_out][P]
    int64_t M, N, O, P;
    int64_t rows_out;     // rows of each split in `part`
    int64_t row_blocks;   // row tiles used for the unit mapping
    int splits;
    int act1;
    int cus;              // compute units of the device (grouped form: tail splitting)
    bool part_wt;         // partials written through to the memory-side cache (sc1)
    GroupedRows g;
};

// Partial stores.  Partials that fit the 256 MB memory-side cache (the MALL)
// are written through to it at device scope (sc1), so the reduction that
// follows reads most of them from there; larger ones are streamed past the
// caches (non-temporal).  Measured on MI355X (kernel + reduction, us): prefill
// shard, 256 MiB of partials: 166 + 54 streamed, 168 + 44 written through
// (SwiGLU shard: 230 + 55, 233 + 45; expert-sharded MoE, 128 MiB: kernel 140,
// 137); large shard, 2 GiB: 1307 + 429 streamed, 1480 + 472 written through;
// MoE, 512 MiB: 488 streamed, 510 written through.
constexpr int64_t kMallBytes = 256ll << 20;
constexpr int64_t kL2Bytes = 4ll << 20;   // L2 of one XCD
constexpr int64_t kPassWindow = 4;        // pass rotation window when W2's block overflows it
constexpr int kWideChunk = 896;           // dense two-pass chunk: 448 + 448 hidden columns
constexpr int64_t kRoundUnits = 256;      // workgroups in one round on MI355X (one per CU)
constexpr int kCpolSc1 = 16;   // buffer cache-policy bits: sc1 (device scope)
constexpr int kCpolNt = 2;     // ... nt (streaming)
typedef unsigned uint32x3_t __attribute__((ext_vector_type(3)));
typedef unsigned uint32x4_t __attribute__((ext_vector_type(4)));

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

// Grouped form: the same XCD-aware split mapping, but XCD x takes a block of
// consecutive row tiles (x / splits selects the block) instead of every
// (8/splits)-th tile, so the 32 units an XCD runs at once are consecutive
// tiles of the heaviest-first table and span fewer experts' weight chunks in
// its L2 (MoE workload: grouped kernel 504.5 -> 495 us; the dense form measured
// 151.4 -> 153 us with it and keeps map_unit).  `row_blocks` must be a
// multiple of 8 / splits.
__device__ __forceinline__ void map_unit_blocked(int64_t unit, int64_t row_blocks, int splits,
                                                 int64_t* rb, int* s) {
    const int g = 8 / splits;
    const int x = (int)(unit & 7);
    const int64_t j = unit >> 3;
    *s = x % splits;
    *rb = (int64_t)(x / splits) * (row_blocks / g) + j;
}

// What both roles of a first-product pass share.
struct G1Ctx {
    char* smem;
    int32x4_t rx;        // X rows of the tile
    uint32_t xrow_off;   // this loader lane's X row (kOOB past the valid rows)
    uint32_t w1_lane;    // this lane's slot offset inside a W1 block
    int64_t N, O, nk, nk2, rot1;
    int w4, xc, lane;
};

// Both products run the same pipeline, split between two kinds of wave.  The
// four loader waves only issue direct global->LDS loads; the four multiplier
// waves only read LDS and issue MFMAs.  Each SIMD holds one wave of each kind,
// so a loader stalled on the address unit never holds back the matrix core.
// The LDS ring holds NS stages; the loaders run NS-1 stages ahead.  At the top
// of every iteration the loaders wait until their loads of the current stage
// have landed, one barrier publishes the stage and releases the buffer read in
// the previous iteration, then the loaders refill that buffer while the
// multipliers work on the current one.  Loads past the end of K are never
// issued; the last iterations wait for every load still in flight instead.
// The two roles run separate loops that execute the same number of barriers
// per pass: nk2 + 2.

// Loader side of one pass.  rw1 / rw1u start at the pass's first gate / up
// column (dense form: rw1 at the first W1 column; rw1u unused).
template <class PC, bool kGated>
__device__ __forceinline__ void gemm1_loads(const G1Ctx& c, int32x4_t rw1, int32x4_t rw1u) {
    // loads of the i-th stage in walking order (K stage (i + rot1) mod nk); the
    // padding stage i == nk of an odd stage count reads zeros
    auto issue1 = [&](int64_t i, int buf) {
        const bool real = i < c.nk;
        const int64_t kt = !real ? 0 : (i + c.rot1 < c.nk ? i + c.rot1 : i + c.rot1 - c.nk);
        char* st = c.smem + buf * PC::kStage1;
        const int64_t kx = kt * kBK + 8 * c.xc;
        dma16(c.rx, real && kx < c.N ? c.xrow_off + (uint32_t)(kx * 2) : kOOB, st + c.w4 * kFrag);
#pragma unroll
        for (int b = 0; b < PC::kNB1; ++b) {
            const int blk = c.w4 + kMulWaves * b;
            const int r = blk / PC::kNB1, cb = blk % PC::kNB1;
            // gated form: blocks cb < kNB1/2 hold gate columns, the rest the up
            // columns of the same hidden indices
            const bool up = kGated && cb >= PC::kNB1 / 2;
            const int cc = up ? cb - PC::kNB1 / 2 : cb;
            const uint32_t base = (uint32_t)(((kt * kBK + 8 * r) * c.O + 64 * cc) * 2);
            dma16(up ? rw1u : rw1, real ? base + c.w1_lane : kOOB, st + kSub + blk * kFrag);
        }
    };
#pragma unroll
    for (int i = 0; i < PC::kNS1 - 1; ++i)
        if (i < c.nk2) issue1(i, i);
    // barrier -1 publishes stage 0; barrier kt publishes stage kt + 1 (the
    // multipliers read one stage ahead of the one they multiply)
    if (PC::kNS1 - 2 < c.nk2) wait_vmcnt<PC::kD1 * (PC::kNS1 - 2)>();
    else wait_vmcnt<0>();
    __syncthreads();
    int ibuf = PC::kNS1 - 1;
    for (int64_t kt = 0; kt < c.nk2; ++kt) {
        // stages kt+1 .. min(kt + NS1 - 2, nk2 - 1) may be in flight
        if (kt + PC::kNS1 - 2 < c.nk2) wait_vmcnt<PC::kD1 * (PC::kNS1 - 3)>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (kt + PC::kNS1 - 1 < c.nk2) issue1(kt + PC::kNS1 - 1, ibuf);
        ibuf = (ibuf + 1 == PC::kNS1) ? 0 : ibuf + 1;
    }
    __syncthreads();   // the multipliers are done with the ring
}

// Loader side of one pass, register-staged form: each lane loads its 16-byte
// pieces of a stage (the same pieces, with the same offsets, as the direct
// loads above) into registers two stages ahead, and writes them into the LDS
// slot the direct load would fill just before the barrier that publishes the
// stage.  The same barriers as the direct form, in the same places.
template <class PC, bool kGated>
__device__ __forceinline__ void gemm1_loads_reg(const G1Ctx& c, __amdgpu_buffer_rsrc_t rx,
                                                __amdgpu_buffer_rsrc_t rw1,
                                                __amdgpu_buffer_rsrc_t rw1u) {
    auto load = [&](int64_t i, uint4 (&r)[PC::kD1]) {
        const bool real = i < c.nk;
        const int64_t kt = !real ? 0 : (i + c.rot1 < c.nk ? i + c.rot1 : i + c.rot1 - c.nk);
        const int64_t kx = kt * kBK + 8 * c.xc;
        r[0] = bload16(rx, real && kx < c.N ? c.xrow_off + (uint32_t)(kx * 2) : kOOB);
#pragma unroll
        for (int b = 0; b < PC::kNB1; ++b) {
            const int blk = c.w4 + kMulWaves * b;
            const int rr = blk / PC::kNB1, cb = blk % PC::kNB1;
            const bool up = kGated && cb >= PC::kNB1 / 2;
            const int cc = up ? cb - PC::kNB1 / 2 : cb;
            const uint32_t base = (uint32_t)(((kt * kBK + 8 * rr) * c.O + 64 * cc) * 2);
            r[1 + b] = bload16(up ? rw1u : rw1, real ? base + c.w1_lane : kOOB);
        }
    };
    auto store = [&](int64_t i, const uint4 (&r)[PC::kD1]) {
        char* st = c.smem + (int)(i % PC::kNS1) * PC::kStage1;
        *reinterpret_cast<uint4*>(st + c.w4 * kFrag + 16 * c.lane) = r[0];
#pragma unroll
        for (int b = 0; b < PC::kNB1; ++b) {
            const int blk = c.w4 + kMulWaves * b;
            *reinterpret_cast<uint4*>(st + kSub + blk * kFrag + 16 * c.lane) = r[1 + b];
        }
    };
    // Every load is issued, also those of the stages past the end (their
    // offsets are out of range: they read zeros and touch no memory), so the
    // load sequence is the same on every iteration and each register set's
    // wait counts only the loads issued after it.  The stage written after the
    // last one (index nk2) lands in a buffer the multipliers no longer use.
    uint4 RA[PC::kD1], RB[PC::kD1];   // stages of even / odd index
    load(0, RA);
    load(1, RB);
    store(0, RA);
    load(2, RA);
    __syncthreads();   // barrier -1 publishes stage 0
    // iteration kt: stage kt + 1 is written and published by barrier kt, then
    // the registers it used take stage kt + 3
    for (int64_t kt = 0; kt < c.nk2; kt += 2) {
        store(kt + 1, RB);
        __syncthreads();
        load(kt + 3, RB);
        store(kt + 2, RA);
        __syncthreads();
        load(kt + 4, RA);
    }
    __syncthreads();   // the multipliers are done with the ring
}

// Multiplier side of one pass: A^T = W1_pass^T X^T into acc[fo][fm] (hidden
// fragment w4 + 4 fo, row fragment fm).
template <class PC>
__device__ __forceinline__ void gemm1_mma(const G1Ctx& c, floatx4_t (&acc)[PC::kFO][4]) {
    const int li = c.lane & 15, lg = c.lane >> 4;
#pragma unroll
    for (int i = 0; i < PC::kFO; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    const int xoff = 16 * xfrag_slot(li, lg);
    // multiplier w owns hidden fragments w, w+4, w+8, ...: f % 4 == w
    const uint32_t trw1 = wtile_tr_base(c.lane, PC::kNB1, c.w4);
    // Software pipeline: after barrier kt (which publishes stage kt+1) the
    // multiplier reads stage kt+1 while it multiplies stage kt from registers
    // read one iteration earlier.  The reads are spread over the MFMAs (the X
    // fragments first, then one W fragment ahead of each group of four MFMAs),
    // so the LDS sees a steady stream and its latency hides behind the matrix
    // work.  A read past the last stage fetches a stale buffer that is never
    // multiplied.
    auto step = [&](int buf, uint4 (&xn)[4], uint4 (&wn)[PC::kFO], const uint4 (&xcur)[4],
                    const uint4 (&wcur)[PC::kFO]) {
        const char* st = c.smem + buf * PC::kStage1;
        const char* sw = st + kSub + trw1;
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) xn[fm] = ld16(st + fm * kFrag + xoff);
#pragma unroll
        for (int fo = 0; fo < PC::kFO; ++fo) {
            const uint2 lo = lds_read_tr16(sw + 1024 * fo);
            const uint2 hi = lds_read_tr16(sw + 1024 * fo + 512);
            wn[fo] = make_uint4(lo.x, lo.y, hi.x, hi.y);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int fm = 0; fm < 4; ++fm)
                acc[fo][fm] = mfma16x16x32(wcur[fo], xcur[fm], acc[fo][fm]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    uint4 xa[4], wa[PC::kFO], xb[4], wb[PC::kFO];
    __syncthreads();
    {
        const char* st = c.smem;
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) xa[fm] = ld16(st + fm * kFrag + xoff);
#pragma unroll
        for (int fo = 0; fo < PC::kFO; ++fo) {
            const uint2 lo = lds_read_tr16(st + kSub + trw1 + 1024 * fo);
            const uint2 hi = lds_read_tr16(st + kSub + trw1 + 1024 * fo + 512);
            wa[fo] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
    }
    int rbuf = 1;
    for (int64_t kt = 0; kt < c.nk2; kt += 2) {
        __syncthreads();
        step(rbuf, xb, wb, xa, wa);
        rbuf = (rbuf + 1 == PC::kNS1) ? 0 : rbuf + 1;
        __syncthreads();
        step(rbuf, xa, wa, xb, wb);
        rbuf = (rbuf + 1 == PC::kNS1) ? 0 : rbuf + 1;
    }
    __syncthreads();   // every multiplier is done with the ring
}

// Epilogue of one pass: H = act(A + b1) (gated: silu(gate) * up) -> bf16 ->
// LDS slabs from `hs` on, in the GEMM2 operand layout.  og0 is the global
// hidden index of the pass's first column; columns at or past O become zero.
// Gated form: fragment fo (< kFO/2) holds gate columns and fragment fo + kFO/2
// the up columns of the same hidden indices (block fo of the W1 stage is
// fragment fo of every wave).  Both forms round H to bf16 once; with kHLo the
// residue h - bf16(h), rounded to bf16, goes kLoOff bytes further.
template <class PC, bool kGated, bool kHLo, int kLoOff>
__device__ __forceinline__ void gemm1_epilogue(const floatx4_t (&acc)[PC::kFO][4], char* hs,
                                               int64_t og0, int64_t O, const uint16_t* b1,
                                               int act1, int w4, int lane) {
    const int li = lane & 15, lg = lane >> 4;
#pragma unroll
    for (int fo = 0; fo < (kGated ? PC::kFO / 2 : PC::kFO); ++fo) {
        const int ol = 16 * (w4 + kMulWaves * fo) + 4 * lg;  // first of 4 hidden cols
        const int64_t og = og0 + ol;
        float bias[4] = {0.f, 0.f, 0.f, 0.f};
        const bool colok = og < O;  // O % 8 == 0, so the 4 columns are all in or all out
        if (!kGated && colok && b1) {
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
            for (int r = 0; r < 4; ++r) {
                if constexpr (kGated)
                    h[r] = colok ? silu(acc[fo][fm][r]) * acc[fo + PC::kFO / 2][fm][r] : 0.f;
                else
                    h[r] = colok ? apply_act(act1, acc[fo][fm][r] + bias[r]) : 0.f;
            }
            const uint2 pk = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
            char* dst = hs + slab * kSub + frag_off(16 * fm + li, g) + 2 * e;
            *reinterpret_cast<uint2*>(dst) = pk;
            if constexpr (kHLo) {
                // h - hi is exact in fp32 (hi is h rounded to 8 significant bits)
                const uint2 lo = make_uint2(pack_bf16x2(h[0] - bf16_lo(pk.x), h[1] - bf16_hi(pk.x)),
                                            pack_bf16x2(h[2] - bf16_lo(pk.y), h[3] - bf16_hi(pk.y)));
                *reinterpret_cast<uint2*>(dst + kLoOff) = lo;
            }
        }
    }
}

template <int CA, int CB, bool kGrouped, bool kGated, bool kHLo>
__global__ __launch_bounds__(kThreads, 1) void fused_ffn_bf16_kernel(FusedArgs a) {
    using Cfg = FusedCfg<CA, CB, kGated, kHLo>;
    using PA = typename Cfg::PA;
    using PB = typename Cfg::PB;
    static_assert(!(kGrouped && kGated), "the grouped form is not gated");
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool loader = wave >= kMulWaves;   // wave-uniform role
    const int w4 = wave & (kMulWaves - 1);   // index within the role
    const int li = lane & 15;   // fragment index
    const int lg = lane >> 4;   // fragment k-group

    // GEMM2 passes: 1024 output columns where P is a multiple of 128 (the
    // 16-byte form of the second product), else 512
    const int64_t pass_cols = a.P % 128 == 0 ? 1024 : kBN2;
    const int64_t np = (a.P + pass_cols - 1) / pass_cols;
    int64_t rb;
    int s;
    int64_t pass0 = 0, npl = np;   // GEMM2 passes of this workgroup: pass0 .. pass0 + npl - 1
    if constexpr (kGrouped) {
        // The unit count (tiles x splits) is known only on the device.  Units
        // fill whole rounds of `cus` workgroups; a short last round would leave
        // most of the chip idle for a whole unit time, so each of its units is
        // cut into f pieces (f a power of two dividing the pass count, f <=
        // cus / tail): every piece recomputes the unit's H and runs 1/f of the
        // GEMM2 passes.  The grid has cus + 64 workgroups beyond the unit bound.
        // (Measured on the MoE workload: 541 -> 526 us.  A persistent form
        // taking units from per-XCD queues measured 533 us.)
        const int64_t U = (int64_t)(*a.g.tile_count) * a.splits;
        const int64_t full = U / a.cus * a.cus;
        const int64_t w = blockIdx.x;
        if (w < full) {
            // the XCD-aware order covers whole rounds exactly when they hold a
            // multiple of 8 units; the blocked form numbers the full rounds'
            // units (full / splits row tiles) one to one
            if (a.cus % 8 == 0 && 8 % a.splits == 0 && (full / a.splits) % (8 / a.splits) == 0) {
                map_unit_blocked(w, full / a.splits, a.splits, &rb, &s);
            } else if (a.cus % 8 == 0) {
                map_unit(w, a.row_blocks, a.splits, &rb, &s);
            } else {
                rb = w / a.splits;
                s = (int)(w % a.splits);
            }
        } else {
            const int64_t tail = U - full;
            int64_t f = 1;
            while (f < 8 && tail * f * 2 <= a.cus && np % (f * 2) == 0) f *= 2;
            // the f pieces of tail unit t run on one XCD (workgroup index = t
            // mod 8), so they share the unit's W1 chunk and X rows in that L2
            const int64_t j = w - full;
            const int64_t q = j >> 3;
            const int64_t t = (j & 7) + 8 * (q / f);
            if (t >= tail) return;
            const int64_t u = full + t;
            rb = u / a.splits;
            s = (int)(u % a.splits);
            npl = np / f;
            pass0 = (q % f) * npl;
        }
    } else {
        map_unit(blockIdx.x, a.row_blocks, a.splits, &rb, &s);
    }

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
    const int64_t o0 = (int64_t)s * Cfg::kHid;
    const int64_t oc = (O - o0) < Cfg::kHid ? (O - o0) : Cfg::kHid;  // valid hidden columns of this chunk

    G1Ctx c;
    c.smem = smem;
    c.N = N;
    c.O = O;
    c.w4 = w4;
    c.lane = lane;
    // ---- X slab loads: loader w fills fragment w (rows 16w..16w+15); lane l
    // brings row 16w + l/4, k-group xc into fragment slot l (see xfrag_slot).
    const int xr = 16 * w4 + (lane >> 2);
    c.xc = (lane & 3) ^ ((lane >> 3) & 3);
    c.xrow_off = kOOB;
    if constexpr (kGrouped) {
        c.rx = make_srd(a.X, a.M * N * 2);
        if (loader && xr < valid) c.xrow_off = (uint32_t)((a.g.sorted[row0 + xr] / a.g.k) * N * 2);
    } else {
        c.rx = make_srd(a.X + row0 * N, (int64_t)valid * N * 2);
        if (xr < valid) c.xrow_off = (uint32_t)(xr * N * 2);
    }
    // ---- weight loads: lane l brings slot l of a block (see wtile_dma_off).
    // Each W1 resource ends at the end of its matrix, so rows past N read
    // zeros; columns past this chunk's valid width read finite neighbours (or
    // zeros) whose H columns the epilogue forces to zero.
    c.w1_lane = wtile_dma_off(lane, (uint32_t)(O * 2));
    c.nk = (N + kBK - 1) / kBK;
    c.nk2 = (c.nk + 1) & ~(int64_t)1;   // stages walked, padded to even

    // W2 stage: 32 hidden rows x 512 output columns.  The W2 resource covers
    // exactly this chunk's rows, so rows past the chunk read zeros; columns
    // past P read finite neighbours that reach only unstored partial columns.
    const int64_t nsteps = npl * Cfg::kKS;   // GEMM2 stages; the ring runs across passes
    // Staggered stage order (dense form).  The workgroups of one XCD share the
    // weight chunk; walking it in the same order they would all request the
    // same lines at the same moment and queue on the same L2 channels.
    // Workgroup j of the XCD starts instead at K stage j (wrapping) and at W2
    // stage (j, j) of the (pass, k) grid, so at any moment they read different
    // stages (measured against smaller rotations, j mod 16 .. j mod 2, and
    // against rotating only the k order inside each pass: all slower).  The
    // grouped form walks its passes in plain order: its co-resident
    // workgroups can belong to several experts, and walking each expert's W2
    // in step keeps the L2 footprint to one sliding window per expert (560 ->
    // 530 us on the MoE workload); the k order inside a pass rotates, so that
    // workgroups of one expert read different slabs of the same pass (530 ->
    // 487 us), and with the blocked unit numbering (mostly one expert per XCD
    // at a time) the first product takes the dense form's staggered start
    // too (499 -> 495 us; rotating the passes as well: 508 us).
    // The pass rotation spans every pass only while the chunk's W2 block
    // (hidden columns x P) fits the XCD's 4 MB L2 and stays resident; a larger
    // block is walked by the co-resident workgroups inside a window of 4
    // passes, so the lines they share are still in L2 when the later ones
    // read them (large shard, 448 x 8192 block: kernel 1325 -> ~1150 us, an
    // 8-pass window ~1190; prefill shard, 448 x 4096 block: a window of 4, 2
    // or 1 passes 172-176 us against 155 for the full rotation).
    const int64_t jx = blockIdx.x >> 3;
    c.rot1 = jx % c.nk;
    const int64_t pass_window = kPassWindow * kBN2 / pass_cols;   // 2048 columns
    const int64_t rot_span =
        (int64_t)Cfg::kHid * P * 2 <= kL2Bytes ? npl : (npl < pass_window ? npl : pass_window);
    const int64_t rotp = kGrouped ? 0 : jx % rot_span;
    const int rotk = (int)(jx % Cfg::kKS);
    char* const hreg = smem + Cfg::kHOff;

    if (loader) {
        // A pass whose LDS ring is only three stages deep (the second pass of
        // the dense two-pass chunk) stages its loads through registers: direct
        // loads into a 3-deep ring have one iteration to land, register-staged
        // ones about two (large shard, 8192 x 8192 x 3584 x 8192: kernel 1152 ->
        // 1041-1046 us).  4-deep rings keep the direct loads, which measured
        // faster there (prefill shard 144 against 152 us, MoE 452 against 482
        // us, and the large shard's first pass: 1062 us with both passes
        // register-staged).
        auto pass_loads = [&](auto pc, int64_t oo) {
            using PC = decltype(pc);
            if constexpr (PC::kNS1 == 3) {
                const __amdgpu_buffer_rsrc_t rx = kGrouped ? make_rsrc(a.X, a.M * N * 2)
                    : make_rsrc(a.X + row0 * N, (int64_t)valid * N * 2);
                const __amdgpu_buffer_rsrc_t rw1 = make_rsrc(W1 + oo, (N * O - oo) * 2);
                gemm1_loads_reg<PC, kGated>(c, rx, rw1,
                                            kGated ? make_rsrc(a.W1u + oo, (N * O - oo) * 2) : rw1);
            } else {
                gemm1_loads<PC, kGated>(c, make_srd(W1 + oo, (N * O - oo) * 2),
                                        kGated ? make_srd(a.W1u + oo, (N * O - oo) * 2) : c.rx);
            }
        };
        pass_loads(PA{}, o0);
        if constexpr (Cfg::kTwoPass) pass_loads(PB{}, o0 + Cfg::kHidA);
    } else {
        {
            floatx4_t acc[PA::kFO][4];
            gemm1_mma<PA>(c, acc);
            gemm1_epilogue<PA, kGated, kHLo, Cfg::kLoOff>(acc, hreg + Cfg::kSlabsB * kSub, o0, O, b1,
                                                          a.act1, w4, lane);
        }
        if constexpr (Cfg::kTwoPass) {
            floatx4_t acc[PB::kFO][4];
            gemm1_mma<PB>(c, acc);
            gemm1_epilogue<PB, kGated, kHLo, Cfg::kLoOff>(acc, hreg, o0 + Cfg::kHidA, O, b1, a.act1,
                                                          w4, lane);
        }
    }
    __syncthreads();   // H is complete

    auto hrow = [](int ks) {
        if constexpr (Cfg::kSlabsB == 0) return kBK * ks;
        else return ks < Cfg::kSlabsB ? Cfg::kHidA + kBK * ks : kBK * (ks - Cfg::kSlabsB);
    };
    // Partial stores.  The resource spans this tile's valid rows of the
    // split's plane, so the stores of rows past them fall outside it and are
    // dropped by the range check, and lanes whose columns lie past P store at
    // kOOB; the offsets are relative to the tile, so they stay below 2^31
    // whatever the plane's size.
    char* const part_tile = a.part + ((int64_t)s * a.rows_out + row0) * P * kPartBytes;
    const __amdgpu_buffer_rsrc_t rpart = make_rsrc(part_tile, (int64_t)valid * P * kPartBytes);

    if (P % 128 == 0) {
        // ================== GEMM2, P a multiple of 128: Y_part = H W2_chunk ==================
        // All eight waves, for output widths that are a multiple of 128.
        // Wave m owns columns 128m .. 128m+127 of every 1024-column pass and
        // streams its W2 columns straight into registers with 16-byte loads:
        // lane (i, g) loads, for each k-row 8g + e of a stage, the eight
        // columns 8i .. 8i+7 (the 16 lanes of a k-group read 256 contiguous
        // bytes of a row).  Column q of that 8 x 8 block, transposed out of the
        // registers (four v_perm) just before its MFMAs, is a k-contiguous
        // operand whose index i stands for column 8i + q.  H is the first MFMA
        // operand, so lane (i, g) ends up with rows 16 fm + 4g + r and, over q,
        // the eight consecutive columns 8i .. 8i+7 (24 bytes of packed
        // partials per row), which reach the partial plane through the wave's
        // LDS staging area in whole 16-byte pieces.  16-byte loads carry twice
        // the bytes of 8-byte ones per address-unit instruction: the W2
        // stream alone takes 33 against 52 us per call at the prefill shard,
        // and this form of the second product ~50 against ~68 us
        // (per-workgroup timestamps).  Two stages are in flight while one is
        // multiplied.
        constexpr int64_t kPW = 1024;   // output columns per pass: eight waves of 128
        const int wm = wave;
        const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(W2 + o0 * P, oc * P * 2);
        const uint32_t w2l =
            (uint32_t)(8 * lg) * (uint32_t)(P * 2) + (uint32_t)(128 * wm + 8 * li) * 2u;
        auto load16 = [&](int64_t step, uint4 (&R)[8]) {
            const int64_t pr = step / Cfg::kKS;
            const int kr = (int)(step - pr * Cfg::kKS);
            const int64_t pt = pass0 + (pr + rotp < npl ? pr + rotp : pr + rotp - npl);
            const int ks = kr + rotk < Cfg::kKS ? kr + rotk : kr + rotk - Cfg::kKS;
            const uint32_t base = step < nsteps
                ? (uint32_t)(((int64_t)hrow(ks) * P + pt * kPW) * 2) + w2l : kOOB;
#pragma unroll
            for (int e = 0; e < 8; ++e) R[e] = bload16(rw2, base + (uint32_t)(e * P * 2));
        };
        floatx4_t acc[8][4];   // [operand q][row fragment fm]
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) acc[q][fm] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        // one stage: each operand column is transposed out of R just before its
        // MFMAs (four v_perm), so only one operand is live besides R; R is
        // refilled with stage st + 2 once the stage's MFMAs are issued
        // (compensated H: one register stage, refilled with stage st + 1 -- the
        // doubled MFMA work of a stage covers the load, and the hi and lo H
        // fragments leave no room for a second stage)
        constexpr int kAhead = kHLo ? 1 : 2;
        auto mma = [&](int64_t st, uint4 (&R)[8]) {
            const int64_t pr = st / Cfg::kKS;
            const int kr = (int)(st - pr * Cfg::kKS);
            const int ks = kr + rotk < Cfg::kKS ? kr + rotk : kr + rotk - Cfg::kKS;
            const char* hs = hreg + ks * kSub;
            uint4 bh[4], bl[4];
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) bh[fm] = ld16(hs + frag_off(16 * fm + li, lg));
            if constexpr (kHLo) {
#pragma unroll
                for (int fm = 0; fm < 4; ++fm) bl[fm] = ld16(hs + Cfg::kLoOff + frag_off(16 * fm + li, lg));
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint4 wq = transpose8x8_col(R, q);
#pragma unroll
                for (int fm = 0; fm < 4; ++fm) acc[q][fm] = mfma16x16x32(bh[fm], wq, acc[q][fm]);
                if constexpr (kHLo) {
#pragma unroll
                    for (int fm = 0; fm < 4; ++fm) acc[q][fm] = mfma16x16x32(bl[fm], wq, acc[q][fm]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            load16(st + kAhead, R);
            __builtin_amdgcn_sched_barrier(0);
        };
        uint4 RA[8], RB[8];
        // all of RA's loads before RB's, as in every later iteration: the
        // compiler's waits at the loop head take the strictest of the paths
        // into it, so a prologue with the two sets interleaved would make
        // every iteration wait for both
        load16(0, RA);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!kHLo) load16(1, RB);   // the stage count is even
        __builtin_amdgcn_sched_barrier(0);
        for (int64_t st = 0; st < nsteps; st += 2) {
            mma(st, RA);
            if constexpr (kHLo) mma(st + 1, RA);
            else mma(st + 1, RB);
            if ((st + 2) % Cfg::kKS != 0) continue;
            const int64_t pr = st / Cfg::kKS;
            // pass pr complete: lane (i, g) holds rows 16 fm + 4 g + r, columns
            // c0w + 8 i + q of the wave's segment.  Its 24 bytes of packed
            // partials per row go through the wave's LDS staging area (8 rows at
            // a time), which is read back in 16-byte pieces that follow the rows
            // of the partial plane, so every store writes whole, adjacent pieces.
            const int64_t pt = pass0 + (pr + rotp < npl ? pr + rotp : pr + rotp - npl);
            const int64_t c0w = pt * kPW + 128 * wm;   // P % 128 == 0: all 128 in or all out
            // the row stride passes through an empty asm statement so that the
            // row offsets are formed here, not held across the loop
            uint32_t rowb = (uint32_t)(P * kPartBytes);
            asm volatile("" : "+s"(rowb));
            const uint32_t vo = c0w < P ? (uint32_t)(c0w * kPartBytes) : kOOB;
            char* const stg = smem + Cfg::kStgOff + wm * 3072;
#pragma unroll
            for (int fm = 0; fm < 4; ++fm)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
#pragma unroll
                    for (int rr = 0; rr < 2; ++rr) {
                        const int r = 2 * t + rr;
                        uint32_t w0[3], w1[3];
                        pack_f24x4(acc[0][fm][r], acc[1][fm][r], acc[2][fm][r], acc[3][fm][r], w0);
                        pack_f24x4(acc[4][fm][r], acc[5][fm][r], acc[6][fm][r], acc[7][fm][r], w1);
                        char* dst = stg + (2 * lg + rr) * 384 + 24 * li;
                        *reinterpret_cast<uint2*>(dst) = make_uint2(w0[0], w0[1]);
                        *reinterpret_cast<uint2*>(dst + 8) = make_uint2(w0[2], w1[0]);
                        *reinterpret_cast<uint2*>(dst + 16) = make_uint2(w1[1], w1[2]);
                    }
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        const int cidx = lane + 64 * k;   // 16-byte piece 0..191 of the 8 rows
                        const int ri = cidx / 24, pos = cidx - 24 * (cidx / 24);
                        const uint4 v = *reinterpret_cast<const uint4*>(stg + ri * 384 + pos * 16);
                        const int row = 16 * fm + 4 * (ri >> 1) + 2 * t + (ri & 1);
                        const uint32_t o = vo + (uint32_t)row * rowb + (uint32_t)(pos * 16);
                        if (a.part_wt)   // written through to the MALL
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(uint32x4_t, v), rpart, o, 0, kCpolSc1);
                        else             // streamed: read once, by the reduction
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(uint32x4_t, v), rpart, o, 0, kCpolNt);
                    }
                }
#pragma unroll
            for (int q = 0; q < 8; ++q)
#pragma unroll
                for (int fm = 0; fm < 4; ++fm) acc[q][fm] = floatx4_t{0.f, 0.f, 0.f, 0.f};
        }
        return;
    }

    // ======================= GEMM2: Y_part = H W2_chunk =====================
    // (Output widths that are not a multiple of 128.)  All eight waves.  Wave w owns columns 64w .. 64w+63 of every 512-column
    // pass and streams its own W2 columns straight into registers -- no LDS
    // staging and no barriers.  Lane (i, g) loads, for each k-row 8g..8g+7 of
    // a stage, the four columns 4i..4i+3 (8 bytes: the 16 lanes of a k-group
    // read 128 contiguous bytes of a row).  Eight rows x four columns are
    // transposed in registers into four k-contiguous operands; operand j,
    // index i stands for column 4i + j.  H is the first MFMA operand, so lane
    // (i, g) ends up with rows 16 fm + 4g + r of the four consecutive columns
    // 4i..4i+3 and stores them as one 16-byte write.  H slab ks holds hidden
    // rows hrow(ks) .. +31 of the chunk (pass B's slabs first).
    const int wc = wave;
    const __amdgpu_buffer_rsrc_t rw2 = make_rsrc(W2 + o0 * P, oc * P * 2);
    const uint32_t w2_lane = (uint32_t)(8 * lg) * (uint32_t)(P * 2) + (uint32_t)(64 * wc + 4 * li) * 2u;
    // loads of stage `step` into R; a step past the end reads zeros (out of
    // range), so that every stage refills its registers unconditionally
    auto load2 = [&](int64_t step, uint2 (&R)[8]) {
        const int64_t pr = step / Cfg::kKS;
        const int kr = (int)(step - pr * Cfg::kKS);
        const int64_t pt = pass0 + (pr + rotp < npl ? pr + rotp : pr + rotp - npl);
        const int ks = kr + rotk < Cfg::kKS ? kr + rotk : kr + rotk - Cfg::kKS;
        const uint32_t base = step < nsteps
            ? (uint32_t)(((int64_t)hrow(ks) * P + pt * kBN2) * 2) + w2_lane : kOOB;
#pragma unroll
        for (int e = 0; e < 8; ++e) R[e] = bload8(rw2, base + (uint32_t)(e * P * 2));
    };

    floatx4_t acc2[4][4];   // [operand j][row fragment fm]
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) acc2[j][fm] = floatx4_t{0.f, 0.f, 0.f, 0.f};

    // one stage: H fragments from LDS, W2 operands from the registers loaded
    // two stages earlier (refilled with stage step + 2 once transposed)
    auto mma2 = [&](int64_t step, uint2 (&R)[8]) {
        const int64_t pr = step / Cfg::kKS;
        const int kr = (int)(step - pr * Cfg::kKS);
        const int ks = kr + rotk < Cfg::kKS ? kr + rotk : kr + rotk - Cfg::kKS;
        const char* hs = hreg + ks * kSub;
        uint4 bh[4], bl[4], wop[4];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm) bh[fm] = ld16(hs + frag_off(16 * fm + li, lg));
        if constexpr (kHLo) {
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) bl[fm] = ld16(hs + Cfg::kLoOff + frag_off(16 * fm + li, lg));
        }
        transpose8x4(R, wop);
        __builtin_amdgcn_sched_barrier(0);
        load2(step + 2, R);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) acc2[j][fm] = mfma16x16x32(bh[fm], wop[j], acc2[j][fm]);
        if constexpr (kHLo) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int fm = 0; fm < 4; ++fm) acc2[j][fm] = mfma16x16x32(bl[fm], wop[j], acc2[j][fm]);
        }
    };

    const uint32_t part_lane = (uint32_t)(((4 * lg) * P + 64 * wc + 4 * li) * kPartBytes);
    uint2 RA[8], RB[8];
    load2(0, RA);
    load2(1, RB);   // the stage count is even
    for (int64_t st = 0; st < nsteps; st += 2) {
        mma2(st, RA);
        mma2(st + 1, RB);
        if ((st + 2) % Cfg::kKS != 0) continue;
        // pass complete: lane holds rows 16 fm + 4 lg + r, columns 4 li .. 4 li + 3
        const int64_t pd = st / Cfg::kKS;
        const int64_t pt = pass0 + (pd + rotp < npl ? pd + rotp : pd + rotp - npl);
        // the row stride passes through an empty asm statement so that the
        // sixteen row offsets are formed here, not held across the loop
        uint32_t rowb = (uint32_t)(P * kPartBytes);
        asm volatile("" : "+s"(rowb));
        const uint32_t vo = pt * kBN2 + 64 * wc + 4 * li < P
                                ? part_lane + (uint32_t)(pt * kBN2 * kPartBytes) : kOOB;
        uint32_t w[4][4][3];
#pragma unroll
        for (int fm = 0; fm < 4; ++fm)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pack_f24x4(acc2[0][fm][r], acc2[1][fm][r], acc2[2][fm][r], acc2[3][fm][r], w[fm][r]);
        if (a.part_wt) {   // written through to the MALL
#pragma unroll
            for (int fm = 0; fm < 4; ++fm)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b96(
                        uint32x3_t{w[fm][r][0], w[fm][r][1], w[fm][r][2]}, rpart,
                        vo + (uint32_t)(16 * fm + r) * rowb, 0, kCpolSc1);
        } else {           // streamed: read once, by the reduction
#pragma unroll
            for (int fm = 0; fm < 4; ++fm)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    __builtin_amdgcn_raw_buffer_store_b96(
                        uint32x3_t{w[fm][r][0], w[fm][r][1], w[fm][r][2]}, rpart,
                        vo + (uint32_t)(16 * fm + r) * rowb, 0, kCpolNt);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int fm = 0; fm < 4; ++fm) acc2[j][fm] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
}

// ---------------------------------------------------------------- reduce

// kYF32: fp32 output from fp32 partials (the fp32 path); otherwise bf16 output
// from packed partials (kPartBytes each).
template <bool kYF32, bool kBF32>
__global__ __launch_bounds__(256) void reduce_splits_kernel(const void* __restrict__ part,
                                                            int splits, const void* b2,
                                                            void* Y, int64_t M, int64_t P,
                                                            int act2) {
    const int64_t nvec = M * (P / 8);
    const int64_t split_stride = M * P;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t m = v / (P / 8);
        const int64_t p = (v - m * (P / 8)) * 8;
        float y[8];
        if constexpr (kYF32) {
            const float* src = reinterpret_cast<const float*>(part) + m * P + p;
            float4 lo = *reinterpret_cast<const float4*>(src);
            float4 hi = *reinterpret_cast<const float4*>(src + 4);
            for (int s = 1; s < splits; ++s) {
                const float* q = src + s * split_stride;
                float4 a = *reinterpret_cast<const float4*>(q);
                float4 b = *reinterpret_cast<const float4*>(q + 4);
                lo.x += a.x; lo.y += a.y; lo.z += a.z; lo.w += a.w;
                hi.x += b.x; hi.y += b.y; hi.z += b.z; hi.w += b.w;
            }
            y[0] = lo.x; y[1] = lo.y; y[2] = lo.z; y[3] = lo.w;
            y[4] = hi.x; y[5] = hi.y; y[6] = hi.z; y[7] = hi.w;
        } else {
            const char* src = reinterpret_cast<const char*>(part) + (m * P + p) * kPartBytes;
            load_f24x8(src, y);
            for (int s = 1; s < splits; ++s) {
                float t[8];
                load_f24x8(src + s * split_stride * kPartBytes, t);
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] += t[i];
            }
        }
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

template <int CA, int CB, bool G, bool kGated, bool kHLo = false>
hipError_t launch_fused_impl(const FusedArgs& a, int64_t units, hipStream_t stream) {
    using Cfg = FusedCfg<CA, CB, kGated, kHLo>;
    auto kern = fused_ffn_bf16_kernel<CA, CB, G, kGated, kHLo>;
    static std::atomic<bool> lds_set[kMaxDevices] = {};
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), Cfg::kLdsAll, lds_set);
    if (e != hipSuccess) return e;
    // grouped form: workgroups for the pieces of a short last round (at most
    // cus, plus up to 7 x 8 for the XCD-aligned numbering of the pieces)
    const int64_t grid = units + (G ? a.cus + 64 : 0);
    const int64_t plane_bytes = a.rows_out * a.P * kPartBytes;
    FusedArgs b = a;
    b.part_wt = (int64_t)a.splits * plane_bytes <= kMallBytes;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kThreads), Cfg::kLdsAll, stream, b);
    return hipGetLastError();
}

}  // namespace

int fused_pick_chunk(int64_t O) {
    // prefer an exact chunk whose split count lets every XCD own one chunk
    // (the split count divides 8), then any exact chunk, fewest splits first;
    // a hidden width of at most 256 (an expert's share of a sharded layer)
    // takes the 256-wide chunk instead of half-empty wider ones
    for (int c : {512, 448, 256})
        if (O % c == 0 && 8 % (O / c) == 0) return c;
    if (O % 512 == 0) return 512;
    if (O % 448 == 0) return 448;
    return O <= 256 ? 256 : 512;
}

int fused_num_splits(int64_t O, int chunk) { return (int)((O + chunk - 1) / chunk); }

// Dense form: where 896 hidden columns divide O into a split count that
// divides 8 and the units fill two or more whole rounds of MI355X's 256 CUs,
// each workgroup covers 896 columns in two 448-column first-product passes:
// fewer splits, and fewer partials written and reduced, than any
// single-pass chunk (large shard, 8192 rows x 3584 hidden: 8 splits and 1024
// units of 448 become 4 splits and 512 units).  The rule depends on the shape
// only, so the workspace size is known without a device.
int fused_pick_dense_chunk(int64_t M, int64_t O) {
    const int64_t rows = (M + kBM - 1) / kBM;
    const int64_t s = O / kWideChunk;
    if (O % kWideChunk == 0 && s >= 1 && 8 % s == 0 && rows * s >= 2 * kRoundUnits &&
        (rows * s) % kRoundUnits == 0)
        return kWideChunk;
    return fused_pick_chunk(O);
}

hipError_t launch_fused_bf16(const uint16_t* X, const uint16_t* W1, const uint16_t* b1,
                             const uint16_t* W2, void* part, int64_t M, int64_t N, int64_t O,
                             int64_t P, int act1, int chunk, int64_t row_blocks,
                             int64_t rows_out, const GroupedRows* grouped, hipStream_t stream) {
    FusedArgs a;
    a.X = X;
    a.W1 = W1;
    a.W1u = nullptr;
    a.b1 = b1;
    a.W2 = W2;
    a.part = static_cast<char*>(part);
    a.M = M;
    a.N = N;
    a.O = O;
    a.P = P;
    a.rows_out = rows_out;
    a.row_blocks = row_blocks;
    a.splits = fused_num_splits(O, chunk);
    a.act1 = act1;
    a.cus = device_cus();
    if (grouped) a.g = *grouped;
    const int64_t units = row_blocks * a.splits;
    if (units <= 0) return hipSuccess;
    if (chunk == kWideChunk && !grouped)
        return launch_fused_impl<448, 448, false, false>(a, units, stream);
    if (chunk == 448)
        return grouped ? launch_fused_impl<448, 0, true, false, true>(a, units, stream)
                       : launch_fused_impl<448, 0, false, false>(a, units, stream);
    if (chunk == 256)
        return grouped ? launch_fused_impl<256, 0, true, false, true>(a, units, stream)
                       : launch_fused_impl<256, 0, false, false>(a, units, stream);
    return grouped ? launch_fused_impl<512, 0, true, false, true>(a, units, stream)
                   : launch_fused_impl<512, 0, false, false>(a, units, stream);
}

// Hidden columns per workgroup of the gated kernel: 448 (two passes, 256 +
// 192) or 256 (one pass).  As for the dense chunk: prefer an exact width
// whose split count divides 8, then any exact width, fewest splits first.
int fused_swiglu_hid(int64_t O) {
    constexpr int h2 = FusedCfg<512, 384, true>::kHid, h1 = FusedCfg<512, 0, true>::kHid;
    for (int h : {h2, h1})
        if (O % h == 0 && 8 % (O / h) == 0) return h;
    if (O % h2 == 0) return h2;
    if (O % h1 == 0) return h1;
    return O > h1 ? h2 : h1;
}

int fused_swiglu_splits(int64_t O) {
    const int h = fused_swiglu_hid(O);
    return (int)((O + h - 1) / h);
}

hipError_t launch_fused_swiglu_bf16(const uint16_t* X, const uint16_t* Wg, const uint16_t* Wu,
                                    const uint16_t* Wd, void* part, int64_t M, int64_t N,
                                    int64_t O, int64_t P, hipStream_t stream) {
    FusedArgs a;
    a.X = X;
    a.W1 = Wg;
    a.W1u = Wu;
    a.b1 = nullptr;
    a.W2 = Wd;
    a.part = static_cast<char*>(part);
    a.M = M;
    a.N = N;
    a.O = O;
    a.P = P;
    a.rows_out = M;
    a.row_blocks = (M + kBM - 1) / kBM;
    a.splits = fused_swiglu_splits(O);
    a.act1 = 0;
    a.cus = device_cus();
    const int64_t units = a.row_blocks * a.splits;
    if (units <= 0) return hipSuccess;
    if (fused_swiglu_hid(O) == FusedCfg<512, 384, true>::kHid)
        return launch_fused_impl<512, 384, false, true>(a, units, stream);
    return launch_fused_impl<512, 0, false, true>(a, units, stream);
}

hipError_t launch_reduce_splits(const void* part, int splits, const void* b2, int b2_f32,
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
