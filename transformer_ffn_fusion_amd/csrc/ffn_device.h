// ffn_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Fragment conventions for the CDNA4 bf16 matrix instruction
// v_mfma_f32_16x16x32_bf16 (wave64):
//   operand fragment: lane l supplies 8 bf16 values of row/column (l % 16) for
//     the k-values 8*(l/16) + 0..7 of a 32-deep k-step (A and B use the same
//     lane <-> (index, k) convention, so the dot product is over matching k);
//   result: lane l holds D[4*(l/16) + r][l % 16] for r = 0..3.
//
// LDS operand tiles are stored "fragment-major": for every group of 16
// indices (rows of A, columns of B) and every 8-wide k-group g there is one
// 256-byte line holding the 16 indices' 16-byte k-chunks.  Inside the line the
// chunk slot is XOR-swizzled so that
//   * the MFMA fragment read (16 lanes = 16 consecutive indices, fixed g) and
//   * the transposing writes of weight tiles (lanes spread over k-groups and
//     8-column groups, fixed column offset within the group)
// each touch 16 distinct 16-byte slots of the line: no bank conflicts with
// either 32 or 64 four-byte banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ffn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

enum Act { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };

// ---------------------------------------------------------------- numerics

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even, hardware convert).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = (__bf16)lo;
    __bf16 b = (__bf16)hi;
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated as x * sigmoid(2u) = x / (1 + exp(-2u)), which is the same
// function (0.5 (1 + tanh u) = 1 / (1 + e^{-2u})) and saturates cleanly:
// exp(-2u) -> inf gives -0, exp(-2u) -> 0 gives x.  The reciprocal is the
// hardware approximation (about 1 ulp), far below the bf16 rounding of H.
__device__ __forceinline__ float gelu_tanh(float x) {
    const float k2 = -2.0f * 0.7978845608028654f;  // -2 sqrt(2/pi)
    float u = x * (1.0f + 0.044715f * x * x);
    float e = __expf(k2 * u);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// silu(x) = x sigmoid(x) = x / (1 + exp(-x)) (the SiLU / Swish-1 unit);
// saturates as gelu_tanh does: -0 for very negative x, x for large x.
__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

__device__ __forceinline__ float apply_act(int act, float x) {
    if (act == ACT_RELU) return x > 0.0f ? x : 0.0f;
    if (act == ACT_GELU_TANH) return gelu_tanh(x);
    return x;
}

// ---------------------------------------------------------------- split partials
//
// The fp32 partial sums of Y that the split-O kernels hand to their ordered
// reduction are stored with a 16-bit significand: the upper three bytes of
// the fp32 pattern (the low byte is dropped, i.e. rounded toward zero).  That
// moves a partial by less than 2^-15 of its magnitude -- far below the one
// bf16 rounding of Y that follows -- and cuts the partial traffic, written and
// read back through HBM or the memory-side cache, by a quarter.  Infinities
// and NaNs stay non-finite.  Four values pack into three dwords:
// w0 = a | b << 24, w1 = b >> 8 | c << 16, w2 = c >> 16 | d << 8 (a..d the
// 24-bit codes), formed with funnel shifts straight from the fp32 patterns.
// (Rounding to nearest instead measured 1.5 us slower on the prefill kernel,
// and 10 us slower with a NaN guard: the packing runs inside the second
// product's loop.)
__device__ __forceinline__ float f24_value(uint32_t code) { return __uint_as_float(code << 8); }

__device__ __forceinline__ void pack_f24x4(float a, float b, float c, float d, uint32_t (&w)[3]) {
    const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
    const uint32_t uc = __float_as_uint(c), ud = __float_as_uint(d);
    w[0] = __builtin_amdgcn_alignbit(ub >> 8, ua, 8);    // a >> 8 | (b >> 8) << 24
    w[1] = __builtin_amdgcn_alignbit(uc >> 8, ub, 16);   // b >> 16 | (c >> 8) << 16
    w[2] = __builtin_amdgcn_alignbit(ud >> 8, uc, 24);   // c >> 24 | (d >> 8) << 8
}
__device__ __forceinline__ void unpack_f24x4(uint32_t w0, uint32_t w1, uint32_t w2, float* v) {
    v[0] = f24_value(w0 & 0xffffffu);
    v[1] = f24_value((w0 >> 24) | ((w1 & 0xffffu) << 8));
    v[2] = f24_value((w1 >> 16) | ((w2 & 0xffu) << 16));
    v[3] = f24_value(w2 >> 8);
}
// Eight consecutive packed values (24 bytes, 8-byte aligned) -> floats.
__device__ __forceinline__ void load_f24x8(const char* src, float (&v)[8]) {
    const uint2 a = *reinterpret_cast<const uint2*>(src);
    const uint2 b = *reinterpret_cast<const uint2*>(src + 8);
    const uint2 c = *reinterpret_cast<const uint2*>(src + 16);
    unpack_f24x4(a.x, a.y, b.x, v);
    unpack_f24x4(b.y, c.x, c.y, v + 4);
}

// ---------------------------------------------------------------- MFMA

__device__ __forceinline__ floatx4_t mfma16x16x32(const uint4& a, const uint4& b, floatx4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- LDS layout

// ---------------------------------------------------------------- stage layouts

constexpr int kFrag = 1024;   // bytes of one 16-index x 32-deep operand fragment

// LDS layout of a row-major weight stage (32 k-rows x `cols` columns), filled by
// direct global->LDS loads and read back through the transposing LDS read.
// The stage is cut into 1 KiB blocks of 8 k-rows x 64 columns, block
// (r, c) at (r * cols/64 + c) KiB.  Inside a block the 16-byte unit holding
// row kk (0..7) and 8-column group u (0..7) sits at slot 8kk + (u ^ 2kk mod 8).
// The loading lane l writes slot l, so lanes 8kk..8kk+7 bring the 128
// contiguous bytes of row kk (every aligned lane quad stays inside one 64-byte
// segment: the loads coalesce).  The 16 lanes of one transposing read (4 rows
// x 2 neighbouring 8-column groups, 8 bytes each) land on 16 distinct 8-byte
// bank positions modulo 128 bytes -- no bank conflicts on the read side either.
__host__ __device__ __forceinline__ uint32_t wtile_dma_off(int l, uint32_t row_bytes) {
    const int kk = l >> 3;
    return (uint32_t)kk * row_bytes + 16u * (uint32_t)((l & 7) ^ ((2 * kk) & 7));
}

// Byte offset, inside a weight stage with `nb` 64-column blocks per row group,
// of the 8-byte chunk that lane l of a transposing read supplies for operand
// fragment f (columns 16f..16f+15), half t (k-rows 8g+4t..8g+4t+3), with
// g = l/16, j = (l%16)/4, q = l%4: row 8g + j + 4t, 8-column group 2f + q/2,
// 4-column half q%2.  Written out with the slot rule above this is
//   wtile_tr_base(l, nb, f % 4) + 1024 * (f / 4) + 512 * t,
// so a wave whose fragments share f % 4 needs one offset register.
__host__ __device__ __forceinline__ uint32_t wtile_tr_base(int l, int nb, int fq) {
    const int g = l >> 4, s = l & 15, j = s >> 2, q = s & 3;
    return (uint32_t)(g * nb * kFrag + 128 * j + 16 * (q >> 1) + 8 * (q & 1) + 32 * (fq ^ j));
}

// LDS layout of one X fragment (16 rows x 32 k, 1 KiB): the 16-byte unit of
// row r and 8-deep k-group c sits at slot 4r + (c ^ (r/2 mod 4)).  The loading
// lane l writes slot l, so lanes 4r..4r+3 bring row r's 64 contiguous bytes;
// the operand read (lane l: row l%16, k-group l/16) is conflict-free within
// every group of 8 lanes.
__host__ __device__ __forceinline__ int xfrag_slot(int r, int c) { return 4 * r + (c ^ ((r >> 1) & 3)); }


// Byte offset of the 16-byte k-chunk (index idx, k-group g) inside a
// fragment-major operand tile (see the file comment).
__host__ __device__ __forceinline__ uint32_t frag_off(uint32_t idx, uint32_t g) {
    uint32_t flip = ((idx >> 3) ^ (idx >> 4)) & 1u;
    uint32_t unit = (idx & 15u) ^ (g | (flip << 2));
    return (((idx >> 4) * 4u + g) << 8) + (unit << 4);
}

// ---------------------------------------------------------------- 8x8 transpose

// rows[i] holds 8 bf16 of row i (dword d = elements 2d, 2d+1).  On return
// cols[j] holds the 8 row-values of column j (dword q = rows 2q, 2q+1).
// v_perm_b32 picks bytes from {S0:S1}; selector 0x05040100 yields
// S1.lo16 | S0.lo16 << 16 and 0x07060302 yields S1.hi16 | S0.hi16 << 16.
__device__ __forceinline__ void transpose8x8(const uint4 (&rows)[8], uint4 (&cols)[8]) {
    const uint32_t LO = 0x05040100u;
    const uint32_t HI = 0x07060302u;
    uint32_t c[8][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 a = rows[2 * q];
        const uint4 b = rows[2 * q + 1];
        c[0][q] = __builtin_amdgcn_perm(b.x, a.x, LO);
        c[1][q] = __builtin_amdgcn_perm(b.x, a.x, HI);
        c[2][q] = __builtin_amdgcn_perm(b.y, a.y, LO);
        c[3][q] = __builtin_amdgcn_perm(b.y, a.y, HI);
        c[4][q] = __builtin_amdgcn_perm(b.z, a.z, LO);
        c[5][q] = __builtin_amdgcn_perm(b.z, a.z, HI);
        c[6][q] = __builtin_amdgcn_perm(b.w, a.w, LO);
        c[7][q] = __builtin_amdgcn_perm(b.w, a.w, HI);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) cols[j] = make_uint4(c[j][0], c[j][1], c[j][2], c[j][3]);
}

// Column j of transpose8x8 alone (four v_perm_b32).
__device__ __forceinline__ uint4 transpose8x8_col(const uint4 (&rows)[8], int j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t c[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint4 a = rows[2 * q];
        const uint4 b = rows[2 * q + 1];
        const uint32_t av = (j >> 1) == 0 ? a.x : (j >> 1) == 1 ? a.y : (j >> 1) == 2 ? a.z : a.w;
        const uint32_t bv = (j >> 1) == 0 ? b.x : (j >> 1) == 1 ? b.y : (j >> 1) == 2 ? b.z : b.w;
        c[q] = __builtin_amdgcn_perm(bv, av, sel);
    }
    return make_uint4(c[0], c[1], c[2], c[3]);
}

// rows[e] holds 4 bf16 (columns 0..3) of row e.  On return cols[j] holds the
// 8 bf16 of column j, rows 0..7 in order.
__device__ __forceinline__ void transpose8x4(const uint2 (&rows)[8], uint4 (&cols)[4]) {
    const uint32_t LO = 0x05040100u;
    const uint32_t HI = 0x07060302u;
    uint32_t c[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint2 a = rows[2 * q];
        const uint2 b = rows[2 * q + 1];
        c[0][q] = __builtin_amdgcn_perm(b.x, a.x, LO);
        c[1][q] = __builtin_amdgcn_perm(b.x, a.x, HI);
        c[2][q] = __builtin_amdgcn_perm(b.y, a.y, LO);
        c[3][q] = __builtin_amdgcn_perm(b.y, a.y, HI);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) cols[j] = make_uint4(c[j][0], c[j][1], c[j][2], c[j][3]);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// ---------------------------------------------------------------- LDS transposing read
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, output lane i,
// element j (of 4 bf16) is element (i % 4) of the 8-byte chunk addressed by
// lane 4*j + i/4 of the same group.  Pointing lane s = 4*j + q at the four
// consecutive columns 4q..4q+3 of k-row j turns a row-major [k][col] tile into
// the k-contiguous operand fragment: lane i receives column i, rows 0..3.
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4_t lds_shortx4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ uint2 lds_read_tr16(const char* p) {
    shortx4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4_t*)(p));
    return __builtin_bit_cast(uint2, v);
}

// ---------------------------------------------------------------- buffer loads
//
// Raw buffer loads with the hardware range check: a load whose byte offset is
// at or beyond the resource's size returns zeros and touches no memory.
// Tails (rows past M or N, columns past O or P) are loaded through an offset
// of kOOB, so the load sequence needs no branches.  Callers keep every
// resource below 2^31 bytes, so kOOB plus any row offset stays out of range.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 descriptor word 3 (32-bit data format)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t nbytes) {
    const int n = nbytes > 0x7fffffff ? 0x7fffffff : (nbytes < 0 ? 0 : (int)nbytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRsrcWord3);
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// Direct global -> LDS load: lane l's 16 bytes land at lds_base + 16*l
// (lds_base must be the same for the whole wave; it goes to M0).  The load
// counts in vmcnt.  It is issued through inline assembly on purpose: the
// compiler cannot prove these LDS writes disjoint from the LDS reads of other
// stages and would otherwise wait for every outstanding load before each LDS
// read, which defeats the multi-stage ring.  Ordering is explicit instead:
// wait_vmcnt<n>() plus a workgroup barrier before a stage is read, and
// wait_vmcnt<0>() before the LDS is reused for anything else or the
// workgroup ends.
typedef int int32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int32x4_t make_srd(const void* base, int64_t nbytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const int n = nbytes > 0x7fffffff ? 0x7fffffff : (nbytes < 0 ? 0 : (int)nbytes);
    int32x4_t r;
    r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));  // stride 0
    r.z = __builtin_amdgcn_readfirstlane(n);
    r.w = kRsrcWord3;
    return r;
}

__device__ __forceinline__ void dma16(const int32x4_t& srd, uint32_t byte_off, char* lds_base) {
    const uint32_t m0 = (uint32_t)(uintptr_t)((lds_void_t*)lds_base);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane((int)m0)), "v"(byte_off), "s"(srd)
        : "m0");
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace ffn
