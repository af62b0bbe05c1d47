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
//    j = b / 8) runs on XCD x.  Its waves 0-3 multiply rows [128 j, +128) of
//    X and W1 over slice x's columns and write that K block's fp32 partial;
//    once all 32 K blocks of the slice are in the XCD's L2, the workgroup sums
//    1/32 of the slice's elements over the 32 K blocks in ascending order,
//    adds b1, applies act1 and writes them to H in bf16 (one rounding);
//  * its waves 4-7 load the workgroup's part of W2 (slice x's rows, output
//    columns [128 j, 128 j + 128)) into registers as soon as they start --
//    W2 does not depend on H, so both weights stream from the first
//    microsecond -- then, once slice x of H is complete, multiply it in; the
//    workgroup writes slice x's fp32 partial of those columns of Y;
//  * a second kernel sums the 8 slice partials of Y in ascending slice order,
//    adds b2 and applies act2 (one rounding to bf16).
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
constexpr int kKRows = kDecodeN / kPerXcd;  // layer-1 K rows per workgroup (128)
constexpr int kPCols = kDecodeP / kPerXcd;  // layer-2 output columns per workgroup (128)
constexpr int kSpin = 1 << 20;              // polls before a wait gives up (~1 s)
constexpr int kCpolSc1 = 16;                // buffer cache-policy bits: sc1 (device scope)
// W2's loads start with the kernel (false) or once layer 1's MFMAs are done,
// leaving the first microseconds of bandwidth to W1 (true)
constexpr bool kW2AfterLayer1 = false;
static_assert(kKRows == 4 * 32, "one 32-deep MFMA step per wave of a layer-1 workgroup");
static_assert(kPCols == 128, "a layer-2 workgroup covers one 128-column load block");
static_assert(16 * kPCols / 4 == 2 * kThreads, "one float4 of the slice partial per thread");

struct DecodeArgs {
    const uint16_t* X;
    const uint16_t* W1;
    const uint16_t* b1;
    const uint16_t* W2;
    float* part1;       // [256][16][ox]: K-block partials of layer 1, by (x, j)
    uint16_t* H;        // [16][O]
    float* part2;       // [8][16][P]: slice partials of layer 2
    uint64_t* flags;    // [2][256]: K block written, H columns written
    uint64_t* status;   // == epoch if this call failed a check
    int64_t M, O, P;
    int ox;             // hidden columns per XCD slice (O / 8)
    int act1;
    uint64_t epoch;
};

__device__ __forceinline__ int xcc_id() {
    // HW_REG_XCC_ID (hardware register 20), bits [3:0]: this wave's XCD
    return (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 15u);
}

// Marks this workgroup's step done.  All of its stores must be complete
// (every thread: s_waitcnt vmcnt(0), then a workgroup barrier) before.
__device__ __forceinline__ void set_flag(uint64_t* flag, uint64_t epoch) {
    if (threadIdx.x == 0)
        __hip_atomic_store(flag, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Waits until the 32 flags of one XCD hold `epoch` (wave 0 polls, one flag
// per lane, with device-scope loads that skip the L1).  Returns false if the
// wait expired.
__device__ bool wait_flags(const uint64_t* flags, uint64_t epoch, int* ok_lds) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        bool done = false;
        for (int it = 0; it < kSpin; ++it) {
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

// One workgroup of 8 waves per CU, workgroup b on XCD x = b mod 8 with index
// j = b / 8 there.  Waves 0-3 compute layer 1 of K block j over slice x: wave
// w takes K rows [128 j + 32 w, +32); lane (g, c) loads rows +8g .. +8g+7 of
// the 8 columns 8c .. 8c+7 of each 128-column block of the slice, transposes
// them in registers into the MFMA's k-contiguous operand and multiplies the
// matching X fragment.  Waves 4-7 hold the workgroup's part of W2 (slice x's
// rows, output columns [128 j, +128)): wave 4 + w takes the slice's 32-row K
// steps w and w + 4 (when there is one).  Only waves 0-3 store and then wait
// for their stores (s_waitcnt vmcnt(0)), so those waits never include the W2
// stream of waves 4-7.
__global__ __launch_bounds__(2 * kThreads) void decode_stream_kernel(DecodeArgs a) {
    __shared__ __attribute__((aligned(16))) float red[4 * 16 * 256];
    __shared__ int ok_lds;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int c = lane & 15;
    const bool l1 = wave < 4;   // layer-1 waves; waves 4-7 run layer 2
    const int w = wave & 3;
    const int x = blockIdx.x % kXcds;
    const int j = blockIdx.x / kXcds;
    const int ox = a.ox;
    const int nks = ox / 32;    // 32-row K steps of layer 2 (the slice's rows)
    const int64_t O = a.O;
    const int64_t P = a.P;
    if (xcc_id() != x) fail(a.status, a.epoch);   // the exchange would not be coherent

    uint4 wr[2][8];
    uint4 af = zero16();
    auto load_w2 = [&]() {
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
    };
    if (l1) {
        const int64_t k = (int64_t)j * kKRows + 32 * w + 8 * g;
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.X, a.M * kDecodeN * 2);
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(a.W1, kDecodeN * O * 2);
        af = bload16(rx, c < a.M ? (uint32_t)((c * kDecodeN + k) * 2) : kOOB);
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int cl = cb * 128 + 8 * c;   // column inside the slice
            const int64_t col = (int64_t)x * ox + cl;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                wr[cb][i] = bload16(rw, cl < ox ? (uint32_t)(((k + i) * O + col) * 2) : kOOB);
        }
    } else if (!kW2AfterLayer1) {
        load_w2();
    }

    // ---- layer 1: this K block's share of slice x of X W1
    if (l1) {
        floatx4_t acc[2][8];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            uint4 cv[8];
            transpose8x8(wr[cb], cv);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                acc[cb][q] = mfma16x16x32(af, cv[q], floatx4_t{0.f, 0.f, 0.f, 0.f});
        }
        // acc[cb][q][r] = wave w's share of H[4g + r][cb * 128 + 8c + q]
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float* dst = red + (w * 16 + 4 * g + r) * 256 + cb * 128 + 8 * c;
                *reinterpret_cast<float4*>(dst) =
                    make_float4(acc[cb][0][r], acc[cb][1][r], acc[cb][2][r], acc[cb][3][r]);
                *reinterpret_cast<float4*>(dst + 4) =
                    make_float4(acc[cb][4][r], acc[cb][5][r], acc[cb][6][r], acc[cb][7][r]);
            }
    }
    __syncthreads();
    if (!l1 && kW2AfterLayer1) load_w2();
    if (l1) {
        // the K block's partial: the four waves' 32-row sums added in wave order
        float* mine = a.part1 + (int64_t)(x * kPerXcd + j) * 16 * ox;
        for (int e = 4 * tid; e < 16 * ox; e += 4 * kThreads) {
            const int m = e / ox;
            const int cl = e - m * ox;
            const float* s = red + m * 256 + cl;
            const float4 s0 = *reinterpret_cast<const float4*>(s);
            const float4 s1 = *reinterpret_cast<const float4*>(s + 16 * 256);
            const float4 s2 = *reinterpret_cast<const float4*>(s + 2 * 16 * 256);
            const float4 s3 = *reinterpret_cast<const float4*>(s + 3 * 16 * 256);
            *reinterpret_cast<float4*>(mine + e) =
                make_float4(((s0.x + s1.x) + s2.x) + s3.x, ((s0.y + s1.y) + s2.y) + s3.y,
                            ((s0.z + s1.z) + s2.z) + s3.z, ((s0.w + s1.w) + s2.w) + s3.w);
        }
        wait_vmcnt<0>();
    }
    __syncthreads();
    set_flag(a.flags + x * kPerXcd + j, a.epoch);

    // ---- every K block of slice x is in the L2: finish 1/32 of slice x of H
    // (16 * ox / 32 consecutive elements of the row-major [16][ox] slice, four
    // per thread: each element's 32 K-block partials added in ascending order)
    const bool ok1 = wait_flags(a.flags + x * kPerXcd, a.epoch, &ok_lds);
    if (tid < ox / 8) {   // wave 0: no loads of its own outstanding
        const int e = j * (ox / 2) + 4 * tid;
        const int m = e / ox;
        const int cl = e - m * ox;
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(a.part1 + (int64_t)(x * kPerXcd) * 16 * ox, (int64_t)kPerXcd * 16 * ox * 4);
        float4 t[kPerXcd];
#pragma unroll
        for (int q = 0; q < kPerXcd; ++q)   // written by other CUs: device-scope (sc1) loads
            t[q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rp, (uint32_t)((q * 16 * ox + e) * 4), 0, kCpolSc1));
        float v[4] = {t[0].x, t[0].y, t[0].z, t[0].w};
#pragma unroll
        for (int q = 1; q < kPerXcd; ++q) {
            v[0] += t[q].x;
            v[1] += t[q].y;
            v[2] += t[q].z;
            v[3] += t[q].w;
        }
        const int64_t col = (int64_t)x * ox + cl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (a.b1) v[i] += bf16_to_f32(a.b1[col + i]);
            v[i] = ok1 ? apply_act(a.act1, v[i]) : __builtin_nanf("");
        }
        *reinterpret_cast<uint2*>(a.H + m * O + col) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        wait_vmcnt<0>();
    }
    if (!ok1) fail(a.status, a.epoch);
    __syncthreads();
    set_flag(a.flags + kRoleWgs + x * kPerXcd + j, a.epoch);

    // ---- slice x of H is complete: layer 2 over it
    const bool ok2 = wait_flags(a.flags + kRoleWgs + x * kPerXcd, a.epoch, &ok_lds);
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
    // (16 x 128 values, four per thread)
    {
        const int m = tid / (kPCols / 4);
        const int cl = (tid - m * (kPCols / 4)) * 4;
        const float* s = red + m * 128 + cl;
        const float4 s0 = *reinterpret_cast<const float4*>(s);
        const float4 s1 = *reinterpret_cast<const float4*>(s + 16 * 128);
        const float4 s2 = *reinterpret_cast<const float4*>(s + 2 * 16 * 128);
        const float4 s3 = *reinterpret_cast<const float4*>(s + 3 * 16 * 128);
        float4 v = make_float4(((s0.x + s1.x) + s2.x) + s3.x, ((s0.y + s1.y) + s2.y) + s3.y,
                               ((s0.z + s1.z) + s2.z) + s3.z, ((s0.w + s1.w) + s2.w) + s3.w);
        if (!ok2) v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                  __builtin_nanf(""));
        *reinterpret_cast<float4*>(a.part2 + ((int64_t)x * 16 + m) * P + (int64_t)j * kPCols + cl) = v;
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

DecodeStreamLayout decode_stream_layout(int64_t O, int64_t P) {
    DecodeStreamLayout L;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) & ~(size_t)255;
        return at;
    };
    L.part1 = take(sizeof(float) * kRoleWgs * 16 * (size_t)(O / kXcds));
    L.h = take(sizeof(uint16_t) * 16 * (size_t)O);
    L.part2 = take(sizeof(float) * kXcds * 16 * (size_t)P);
    L.flags = take(sizeof(uint64_t) * 2 * kRoleWgs);
    L.status = take(sizeof(uint64_t));
    L.total = off;
    return L;
}

hipError_t launch_decode_stream(const uint16_t* X, const uint16_t* W1, const uint16_t* b1,
                                const uint16_t* W2, char* ws, int64_t M, int64_t O, int64_t P,
                                int act1, uint64_t epoch, hipStream_t stream) {
    const DecodeStreamLayout L = decode_stream_layout(O, P);
    DecodeArgs a;
    a.X = X;
    a.W1 = W1;
    a.b1 = b1;
    a.W2 = W2;
    a.part1 = reinterpret_cast<float*>(ws + L.part1);
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
    hipLaunchKernelGGL(decode_stream_kernel, dim3(kRoleWgs), dim3(2 * kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_decode_reduce(const uint16_t* b2, uint16_t* Y, char* ws, int64_t M, int64_t O,
                                int64_t P, int act2, uint64_t epoch, hipStream_t stream) {
    const DecodeStreamLayout L = decode_stream_layout(O, P);
    const int64_t nvec = M * (P / 4);
    hipLaunchKernelGGL(decode_reduce_kernel, dim3((unsigned)((nvec + 63) / 64)), dim3(64), 0,
                       stream, reinterpret_cast<const float*>(ws + L.part2),
                       reinterpret_cast<const uint64_t*>(ws + L.status), epoch, b2, Y, M, P, act2);
    return hipGetLastError();
}

}  // namespace ffn
