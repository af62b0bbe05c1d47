// ffn_decode.hip -- the decode-shaped FFN (M <= 16 rows) as one streaming
// kernel and one small reduction, with H exchanged inside each XCD's L2.
//
// Y = act2(act1(X W1 + b1) W2 + b2) (the two equations of the kernel-fusion /
// tensor-parallelism post, brunomaga.github.io, section "Megatron-LM tensor
// parallelism"), for M <= 16 token rows.  At this size the call is a stream
// of W1 and W2 from HBM; what costs time beyond the stream is the chain of
// dependent steps between the two layers.  MI355X has 8 XCDs of 32 CUs, each
// XCD with its own L2; workgroups are dealt to the XCDs in turn
// (workgroup b runs on XCD b mod 8), which every workgroup checks against the
// hardware's XCC_ID register.  The hidden dimension is cut into 8 slices of
// O/8 columns, one per XCD, so that everything layer 2 needs from layer 1
// stays inside one XCD:
//
//  * 256 workgroups of 8 waves, one per CU; workgroup (x, j) (x = b mod 8,
//    j = b / 8) runs on XCD x.  Its waves 0-3 multiply rows [256 (j / 2),
//    +256) of X and W1 over one half (j mod 2) of slice x's columns and write
//    that K block's fp32 partial of the half; once all 16 K blocks of the
//    slice are in the XCD's L2, the workgroup sums 1/32 of the slice's
//    elements over the 16 K blocks in ascending order, adds b1, applies act1
//    and writes them to H in bf16 (one rounding);
//  * its waves 4-7 load the workgroup's part of W2 (slice x's rows, output
//    columns [128 j, 128 j + 128)) into registers as soon as they start --
//    W2 does not depend on H, so both weights stream from the first
//    microsecond -- then, once slice x of H is complete, multiply it in; the
//    workgroup writes slice x's fp32 partial of those columns of Y;
//  * a second kernel sums the 8 slice partials of Y in ascending slice order,
//    adds b2 and applies act2 (one rounding to bf16).
//
// The gated form (SwiGLU: the same post, section "Benchmarks";
// H = silu(X Wg) * (X Wu), no biases) runs 12 waves per workgroup: waves 0-3
// the gate product over Wg, waves 4-7 the up product over Wu (each with its
// own K-block partials), waves 8-11 layer 2 over Wd; the gate and up sums of
// an element meet in one thread, which forms silu(gate) * up before the
// single rounding of H.
//
// The 256 workgroups fit the 256 CUs at once, so the whole grid is resident
// while any of it waits.  Waits are between workgroups of one XCD: a producer's
// stores are complete in the L2 (s_waitcnt vmcnt(0): the L1 is write-through)
// before it sets its flag; a consumer polls the flags, and then reads the
// data behind them, with device-scope loads (sc1), which skip the CU's L1 and
// are served by the XCD's L2 (with group-scope sc0 loads, a poll kept hitting
// the stale line in its own L1 until the wait expired).  No release fence is
// involved (a device-scope release writes back the XCD's L2: ~1.6k cycles on
// this part, serialised within an XCD).  Flags hold the call's epoch (a
// 64-bit number that is new for every call), so nothing has to be cleared
// between calls.
// Every wait is bounded; on expiry, or if a workgroup finds itself on another
// XCD than its number says, the call records its epoch in a status word and
// the reduction writes NaN to all of Y instead of a silently wrong result.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kXcds = 8;
constexpr int kPerXcd = 32;                 // workgroups on one XCD
constexpr int kRoleWgs = kXcds * kPerXcd;   // 256 workgroups in all
constexpr int kThreads = 256;               // threads of the four waves of one role
constexpr int kKBlocks = kPerXcd / 2;       // layer-1 K blocks per slice (two column halves each)
constexpr int kKRows = kDecodeN / kKBlocks; // layer-1 K rows per workgroup (256)
constexpr int kPCols = kDecodeP / kPerXcd;  // layer-2 output columns per workgroup (128)
constexpr int kSpin = 1 << 20;              // polls before a wait gives up (~1 s)
constexpr int kCpolSc1 = 16;                // buffer cache-policy bits: sc1 (device scope)
static_assert(kKRows == 4 * 2 * 32, "two 32-deep MFMA steps per wave of a layer-1 workgroup");
static_assert(kPCols == 128, "a layer-2 workgroup covers one 128-column load block");
static_assert(16 * kPCols / 4 == 2 * kThreads, "one float4 of the slice partial per thread");

struct DecodeArgs {
    const uint16_t* X;
    const uint16_t* W1;   // gated form: the gate matrix Wg
    const uint16_t* W1u;  // gated form: the up matrix Wu
    const uint16_t* b1;
    const uint16_t* W2;
    float* part1;       // [8][16][16][ox]: K-block partials of layer 1, by (x, K block)
    float* part1u;      // gated form: the same for the up product
    uint16_t* H;        // [16][O]
    float* part2;       // [8][16][P]: slice partials of layer 2
    uint64_t* flags;    // [2][256]: K block written, H columns written
    uint64_t* status;   // == epoch if this call failed a check
    int64_t M, O, P;
    int ox;             // hidden columns per XCD slice (O / 8)
    int act1;
    int spin;           // polls before a wait gives up
    uint64_t epoch;
    uint64_t flag_xor;  // 0; nonzero only in the self-test of the expiry path
};

__device__ __forceinline__ int xcc_id() {
    // HW_REG_XCC_ID (hardware register 20), bits [3:0]: this wave's XCD
    return (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 15u);
}

// Marks this workgroup's step done.  All of its stores must be complete
// (every thread: s_waitcnt vmcnt(0), then a workgroup barrier) before.
__device__ __forceinline__ void set_flag(uint64_t* flag, uint64_t value) {
    if (threadIdx.x == 0)
        __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until the 32 flags of one XCD hold `epoch` (wave 0 polls, one flag
// per lane, with device-scope loads that skip the L1).  Returns false if the
// wait expired.
__device__ bool wait_flags(const uint64_t* flags, uint64_t epoch, int spin, int* ok_lds) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        bool done = false;
        for (int it = 0; it < spin; ++it) {
            const uint64_t v = lane < kPerXcd
                                   ? __hip_atomic_load(flags + lane, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT)
                                   : epoch;
            if (__all(v == epoch)) {
                done = true;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (lane == 0) *ok_lds = done ? 1 : 0;
    }
    __syncthreads();
    return *ok_lds != 0;
}

__device__ __forceinline__ void fail(uint64_t* status, uint64_t epoch) {
    if (threadIdx.x == 0)
        __hip_atomic_store(status, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup per CU, workgroup b on XCD x = b mod 8 with index j = b / 8
// there.  The layer-1 waves compute layer 1 of K block j / 2 over half j mod 2
// of slice x: wave w of a group of four takes K rows [256 (j / 2) + 64 w,
// +64) in two 32-row steps; lane (g, c) loads rows +8g .. +8g+7 of each step
// and the 8 columns 8c .. 8c+7 of the half, transposes them in registers into
// the MFMA's k-contiguous operand and multiplies the matching X fragment (a
// 224-column slice has 112-column halves: lanes c = 14, 15 idle).  Plain
// form: waves 0-3 (W1); gated form (SwiGLU, the kernel-fusion post's
// "Benchmarks" section: H = silu(X Wg) * X Wu, no biases): waves 0-3 the gate
// product (Wg), waves 4-7 the up product (Wu).  The last four waves hold the workgroup's part of
// W2 (slice x's rows, output columns [128 j, +128)): wave w of them takes the
// slice's 32-row K steps w and w + 4 (when there is one).  Only layer-1
// waves store and then wait for their stores (s_waitcnt vmcnt(0)), so those
// waits never include the W2 stream of the layer-2 waves.
template <bool kGated>
__global__ __launch_bounds__((kGated ? 3 : 2) * kThreads) void decode_stream_kernel(DecodeArgs a) {
    constexpr int kL1Waves = kGated ? 8 : 4;
    __shared__ __attribute__((aligned(16))) float red[(kGated ? 2 : 1) * 4 * 16 * 256];
    __shared__ int ok_lds;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const bool l1 = wave < kL1Waves;     // layer-1 waves; the last four run layer 2
    const bool up = kGated && wave >= 4 && wave < 8;
    const int w = wave & 3;
    const int x = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    const int ox = a.ox;
    const int nks = ox / 32;    // 32-row K steps of layer 2 (the slice's rows)
    const int64_t O = a.O;
    const int64_t P = a.P;
    float* myred = red + (up ? 4 * 16 * 256 : 0);   // this wave's product's LDS sums
    if (xcc_id() != x) fail(a.status, a.epoch);    // the exchange would not be coherent

    // the elements of H this workgroup finishes after barrier 1: 1/32 of the
    // row-major [16][ox] slice, four consecutive elements per thread of wave 0
    // (gated form: wave 1 sums the up partials of the same elements); their b1
    // values are loaded now, off the chain of dependent steps
    constexpr int kEl = 4;
    const int rt = tid & 63;
    const bool rsum = rt < ox / (2 * kEl) && (wave == 0 || (kGated && wave == 1));
    const int e = j * (ox / 2) + kEl * rt;
    const int hm = e / ox;                                  // row of H
    const int64_t hcol = (int64_t)x * ox + (e - hm * ox);   // first column of H
    float bias[kEl] = {0.f, 0.f, 0.f, 0.f};
    if (!kGated && rsum && wave == 0 && a.b1) {
#pragma unroll
        for (int i = 0; i < kEl; ++i) bias[i] = bf16_to_f32(a.b1[hcol + i]);
    }

    uint4 wr[2][8];
    uint4 af[2] = {zero16(), zero16()};
    const int kb = j >> 1;           // layer 1: K block of kKRows rows ...
    const int hh = j & 1;            // ... and column half of the slice
    const int hw = ox / 2;           // columns of a half
    if (l1) {
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, a.M * kDecodeN * 2);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(up ? a.W1u : a.W1, kDecodeN * O * 2);
        const int cl = hh * hw + 8 * c;
        const int64_t col = (int64_t)x * ox + cl;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int64_t k = (int64_t)kb * kKRows + 64 * w + 32 * s + 8 * g;
            af[s] = bload16(rx, c < a.M ? (uint32_t)((c * kDecodeN + k) * 2) : kOOB);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wr[s][i] = bload16(rw, 8 * c < hw ? (uint32_t)(((k + i) * O + col) * 2) : kOOB);
        }
    } else {
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.W2, O * P * 2);
        const int64_t col = (int64_t)j * kPCols + 8 * c;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ks = w + 4 * s;
            const int64_t n = (int64_t)x * ox + 32 * ks + 8 * g;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wr[s][i] = bload16(rw, ks < nks ? (uint32_t)(((n + i) * P + col) * 2) : kOOB);
        }
    }

    // ---- layer 1: this K block's share of slice x of X W1 (gated: of X Wg and X Wu)
    if (l1) {
        floatx4_t acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            uint4 cv[8];
            transpose8x8(wr[s], cv);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = mfma16x16x32(af[s], cv[q], acc[q]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float* dst = myred + (w * 16 + 4 * g + r) * 256 + 8 * c;
            *reinterpret_cast<float4*>(dst) =
                make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
            *reinterpret_cast<float4*>(dst + 4) =
                make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
        }
    }
    __syncthreads();
    if (l1) {
        // the K block's partial of the half: the four waves' 64-row sums added
        // in wave order
        float* mine = (up ? a.part1u : a.part1) + (int64_t)(x * kKBlocks + kb) * 16 * ox + hh * hw;
        for (int e = 4 * (tid & (kThreads - 1)); e < 16 * hw; e += 4 * kThreads) {
            const int m = e / hw;
            const int cl = e - m * hw;
            const float* s = myred + m * 256 + cl;
            const float4 s0 = *reinterpret_cast<const float4*>(s);
            const float4 s1 = *reinterpret_cast<const float4*>(s + 16 * 256);
            const float4 s2 = *reinterpret_cast<const float4*>(s + 2 * 16 * 256);
            const float4 s3 = *reinterpret_cast<const float4*>(s + 3 * 16 * 256);
            *reinterpret_cast<float4*>(mine + m * ox + cl) =
                make_float4(((s0.x + s1.x) + s2.x) + s3.x, ((s0.y + s1.y) + s2.y) + s3.y,
                            ((s0.z + s1.z) + s2.z) + s3.z, ((s0.w + s1.w) + s2.w) + s3.w);
        }
        wait_vmcnt<0>();
    }
    __syncthreads();
    set_flag(a.flags + x * kPerXcd + j, a.epoch ^ a.flag_xor);

    // ---- every K block of slice x is in the L2: finish this workgroup's
    // elements of H (each element's 16 K-block partials added in ascending
    // order; gated: wave 0 sums the gate partials, wave 1 the up partials)
    const bool ok1 = wait_flags(a.flags + x * kPerXcd, a.epoch, a.spin, &ok_lds);
    {
        typedef float vec_t __attribute__((ext_vector_type(kEl)));
        vec_t v = {};
        if (rsum) {
            const float* src = wave == 1 ? a.part1u : a.part1;
            const __amdgpu_buffer_rsrc_t rp = make_rsrc(src + (int64_t)(x * kKBlocks) * 16 * ox,
                                                        (int64_t)kKBlocks * 16 * ox * 4);
            vec_t t[kKBlocks];
#pragma unroll
            for (int q = 0; q < kKBlocks; ++q) {   // written by other CUs: device-scope (sc1) loads
                const uint32_t off = (uint32_t)((q * 16 * ox + e) * 4);
                t[q] = __builtin_bit_cast(
                    vec_t, __builtin_amdgcn_raw_buffer_load_b128(rp, off, 0, kCpolSc1));
            }
            v = t[0];
#pragma unroll
            for (int q = 1; q < kKBlocks; ++q) v += t[q];
        }
        if constexpr (kGated) {
            // the up sums go to wave 0 through LDS (red is free again: every
            // layer-1 wave finished reading it before the flag above)
            if (rsum && wave == 1) *reinterpret_cast<vec_t*>(red + kEl * rt) = v;
            __syncthreads();
        }
        if (rsum && wave == 0) {
            float h[kEl];
            if constexpr (kGated) {
                const vec_t u = *reinterpret_cast<const vec_t*>(red + kEl * rt);
#pragma unroll
                for (int i = 0; i < kEl; ++i) h[i] = ok1 ? silu(v[i]) * u[i] : __builtin_nanf("");
            } else {
#pragma unroll
                for (int i = 0; i < kEl; ++i)
                    h[i] = ok1 ? apply_act(a.act1, v[i] + bias[i]) : __builtin_nanf("");
            }
            uint32_t* dst = reinterpret_cast<uint32_t*>(a.H + hm * O + hcol);
#pragma unroll
            for (int i = 0; i < kEl / 2; ++i) dst[i] = pack_bf16x2(h[2 * i], h[2 * i + 1]);
            wait_vmcnt<0>();
        }
    }
    if (!ok1) fail(a.status, a.epoch);
    __syncthreads();
    set_flag(a.flags + kRoleWgs + x * kPerXcd + j, a.epoch ^ a.flag_xor);

    // ---- slice x of H is complete: layer 2 over it
    const bool ok2 = wait_flags(a.flags + kRoleWgs + x * kPerXcd, a.epoch, a.spin, &ok_lds);
    if (!l1) {
        const __amdgpu_buffer_rsrc_t rh = make_rsrc(a.H, 16 * O * 2);
        floatx4_t acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ks = w + 4 * s;
            const int64_t hk = (int64_t)x * ox + 32 * ks + 8 * g;
            // H was written by other CUs: a device-scope (sc1) load
            const uint4 hf = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(
                           rh, ks < nks ? (uint32_t)((c * O + hk) * 2) : kOOB, 0, kCpolSc1));
            uint4 cv[8];
            transpose8x8(wr[s], cv);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] = mfma16x16x32(hf, cv[q], acc[q]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float* dst = red + (w * 16 + 4 * g + r) * 128 + 8 * c;
            *reinterpret_cast<float4*>(dst) =
                make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
            *reinterpret_cast<float4*>(dst + 4) =
                make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
        }
    }
    __syncthreads();
    // slice x's partial of Y: the four layer-2 waves' sums added in wave order
    // (16 x 128 values, four per thread of the first 512)
    if (tid < 2 * kThreads) {
        const int mm = tid / (kPCols / 4);
        const int cc = (tid - mm * (kPCols / 4)) * 4;
        const float* s = red + mm * 128 + cc;
        const float4 s0 = *reinterpret_cast<const float4*>(s);
        const float4 s1 = *reinterpret_cast<const float4*>(s + 16 * 128);
        const float4 s2 = *reinterpret_cast<const float4*>(s + 2 * 16 * 128);
        const float4 s3 = *reinterpret_cast<const float4*>(s + 3 * 16 * 128);
        float4 y = make_float4(((s0.x + s1.x) + s2.x) + s3.x, ((s0.y + s1.y) + s2.y) + s3.y,
                               ((s0.z + s1.z) + s2.z) + s3.z, ((s0.w + s1.w) + s2.w) + s3.w);
        if (!ok2) y = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                  __builtin_nanf(""));
        float* dst = a.part2 + ((int64_t)x * 16 + mm) * P + (int64_t)j * kPCols + cc;
        *reinterpret_cast<float4*>(dst) = y;
    }
    if (!ok2) fail(a.status, a.epoch);
}

// Y[m][p] = act2(sum over slices x ascending of part2[x][m][p] + b2[p]), NaN
// for every element if the streaming kernel of this call failed a check.
__global__ __launch_bounds__(64) void decode_reduce_kernel(const float* __restrict__ part2,
                                                           const uint64_t* __restrict__ status,
                                                           uint64_t epoch,
                                                           const uint16_t* __restrict__ b2,
                                                           uint16_t* __restrict__ Y, int64_t M,
                                                           int64_t P, int act2) {
    const int64_t nvec = M * (P / 4);
    const int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (v >= nvec) return;
    const int64_t m = v / (P / 4);
    const int64_t p = (v - m * (P / 4)) * 4;
    float4 t[kXcds];
#pragma unroll
    for (int x = 0; x < kXcds; ++x)
        t[x] = *reinterpret_cast<const float4*>(part2 + ((int64_t)x * 16 + m) * P + p);
    float y[4] = {t[0].x, t[0].y, t[0].z, t[0].w};
#pragma unroll
    for (int x = 1; x < kXcds; ++x) {
        y[0] += t[x].x;
        y[1] += t[x].y;
        y[2] += t[x].z;
        y[3] += t[x].w;
    }
    if (b2) {
        const uint2 bb = *reinterpret_cast<const uint2*>(b2 + p);
        y[0] += bf16_lo(bb.x);
        y[1] += bf16_hi(bb.x);
        y[2] += bf16_lo(bb.y);
        y[3] += bf16_hi(bb.y);
    }
    const bool bad = *status == epoch;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = bad ? __builtin_nanf("") : apply_act(act2, y[i]);
    *reinterpret_cast<uint2*>(Y + m * P + p) =
        make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
}

}  // namespace

bool decode_stream_shape(int64_t M, int64_t N, int64_t O, int64_t P) {
    return M >= 1 && M <= kSkinnyMaxM && N == kDecodeN && P == kDecodeP && O % 256 == 0 &&
           O >= 256 && O <= 2048;
}

DecodeStreamLayout decode_stream_layout(int64_t O, int64_t P, bool gated) {
    DecodeStreamLayout L;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    const size_t part1 = sizeof(float) * kXcds * kKBlocks * 16 * (size_t)(O / kXcds);
    L.part1 = take(part1);
    L.part1u = gated ? take(part1) : L.part1;
    L.h = take(sizeof(uint16_t) * 16 * (size_t)O);
    L.part2 = take(sizeof(float) * kXcds * 16 * (size_t)P);
    L.flags = take(sizeof(uint64_t) * 2 * kRoleWgs);
    L.status = take(sizeof(uint64_t));
    L.total = off;
    return L;
}

hipError_t launch_decode_stream(const uint16_t* X, const uint16_t* W1, const uint16_t* W1u,
                                const uint16_t* b1, const uint16_t* W2, char* ws, int64_t M,
                                int64_t O, int64_t P, int act1, uint64_t epoch,
                                hipStream_t stream, bool expire) {
    const bool gated = W1u != nullptr;
    const DecodeStreamLayout L = decode_stream_layout(O, P, gated);
    DecodeArgs a;
    a.X = X;
    a.W1 = W1;
    a.W1u = W1u;
    a.b1 = b1;
    a.W2 = W2;
    a.part1 = reinterpret_cast<float*>(ws + L.part1);
    a.part1u = reinterpret_cast<float*>(ws + L.part1u);
    a.H = reinterpret_cast<uint16_t*>(ws + L.h);
    a.part2 = reinterpret_cast<float*>(ws + L.part2);
    a.flags = reinterpret_cast<uint64_t*>(ws + L.flags);
    a.status = reinterpret_cast<uint64_t*>(ws + L.status);
    a.M = M;
    a.O = O;
    a.P = P;
    a.ox = (int)(O / kXcds);
    a.act1 = act1;
    a.epoch = epoch;
    // the expiry self-test: flags that never hold the epoch, waits of 64 polls
    a.spin = expire ? 64 : kSpin;
    a.flag_xor = expire ? 1 : 0;
    if (gated)
        hipLaunchKernelGGL(decode_stream_kernel<true>, dim3(kRoleWgs), dim3(3 * kThreads), 0,
                           stream, a);
    else
        hipLaunchKernelGGL(decode_stream_kernel<false>, dim3(kRoleWgs), dim3(2 * kThreads), 0,
                           stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const uint16_t* b2, uint16_t* Y, char* ws, int64_t M, int64_t O,
                                int64_t P, int act2, uint64_t epoch, bool gated,
                                hipStream_t stream) {
    const DecodeStreamLayout L = decode_stream_layout(O, P, gated);
    const int64_t nvec = M * (P / 4);
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((nvec + 63) / 64)), dim3(64), 0,
                       stream, reinterpret_cast<const float*>(ws + L.part2),
                       reinterpret_cast<const uint64_t*>(ws + L.status), epoch, b2, Y, M, P, act2);
    return hipGetLastError();
}

}  // namespace ffn
