// moe.hip -- routing and combine for the grouped (Mixture-of-Experts) form.
//
// Method: the MoE tile-signalling review (zhongzhuzhou.org), section 2.1
// (the router scores the E experts, the top-k are kept, the output is the
// gate-weighted sum of those experts' outputs) and section 2.2 (step 1
// routing, step 3 expert computation, step 5 weighted reduction; the two
// all-to-all steps exist only across GPUs and have no counterpart here).
// The per-expert row lists follow section 4.2's idea of grouping rows so that
// every output tile belongs to one owner -- on one GPU the owner is simply the
// expert -- and section 4.4's heaviest-first tile order; the tile table plays
// the role of section 4.5's per-tile plan (expert, first row, valid rows).
//
// Readings (the pages leave these open): ties between equal logits go to the
// smaller expert index; slot 0 holds the largest logit; the gate weights are a
// softmax over the k selected logits; each expert's list holds its entries
// t*k+s in ascending token order.  All integer outputs are deterministic.
#include "ffn_device.h"
#include "ffn_internal.h"

namespace ffn {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScatterTokens = 256;   // tokens per workgroup of the scatter
constexpr int kRouterTokens = 16;     // tokens per workgroup of the router form
constexpr int kMaxE = 256;
constexpr int kLogitStage = 8192;     // floats of logits held in LDS per workgroup

// Tokens per top-k workgroup: 16 with the router GEMM; with logits as input,
// the largest power of two <= 256 whose logits fit the LDS stage.
int topk_block_tokens(int64_t E, bool router) {
    if (router) return kRouterTokens;
    int tb = kScatterTokens;
    while (tb > 1 && (int64_t)tb * E > kLogitStage) tb >>= 1;
    return tb;
}

// The k largest logits of one row, in decreasing order.  Insertion into a
// sorted list where an equal logit stays behind the earlier expert: the order
// of repeated strict arg-max (ties to the smaller expert index).
template <int k>
__device__ __forceinline__ void topk_row(const float* row, int E, float (&bv)[k], int (&be)[k]) {
#pragma unroll
    for (int j = 0; j < k; ++j) { bv[j] = 0.f; be[j] = 0; }
    int nf = 0;
    for (int e = 0; e < E; ++e) {
        const float v = row[e];
        int p = 0;   // entries that stay ahead: larger or equal logit
#pragma unroll
        for (int j = 0; j < k; ++j) p += (j < nf && bv[j] >= v) ? 1 : 0;
        if (p >= k) continue;
#pragma unroll
        for (int j = k - 1; j > 0; --j)
            if (j > p) { bv[j] = bv[j - 1]; be[j] = be[j - 1]; }
#pragma unroll
        for (int j = 0; j < k; ++j)
            if (j == p) { bv[j] = v; be[j] = e; }
        nf = nf + 1 < k ? nf + 1 : k;
    }
}

struct TopkArgs {
    const float* logits;    // input form: M x E
    const uint16_t* X;      // router form: M x N bf16
    const uint16_t* Wr;     //              N x E bf16 (E % 8 == 0)
    const float* br;        //              E, or null
    float* logits_out;      //              M x E, or null
    int64_t M, N;
    int E;
    int tb;                 // tokens per workgroup
    int32_t* ids;
    float* w;
    int32_t* blk_counts;    // [blocks][E]
};

// Routing step 1 (the review, section 2.2: the gate gives every token its
// expert assignments and gate weights), one block of tokens per workgroup:
// the block's logits into LDS -- read, or computed as X Wr + br (the gate
// read as one linear layer) -- then per token the top-k and the softmax over
// the k selected logits, and the block's expert histogram.
//
// Router form: wave v owns tokens 4v..4v+3 of the block, lane l the k-slices
// 8l + 512i (16-byte loads of X: one wave reads 1 KiB of a row at once), for
// 8 experts at a time; the 64 lanes' partial sums are then added in lane
// order through LDS, so every logit has one fixed summation order.
template <int k, bool kRouter>
__global__ __launch_bounds__(kTopkThreads) void moe_topk_kernel(TopkArgs a) {
    __shared__ float s_log[kLogitStage];
    __shared__ int s_cnt[kMaxE];
    const int tid = threadIdx.x;
    const int E = a.E;
    const int64_t base = (int64_t)blockIdx.x * a.tb;
    const int nb = (a.M - base) < a.tb ? (int)(a.M - base) : a.tb;
    for (int e = tid; e < E; e += kTopkThreads) s_cnt[e] = 0;

    if constexpr (kRouter) {
        __shared__ float s_red[4][32][65];   // [wave][token*8 + expert][lane], padded rows
        const int wv = tid >> 6, kl = tid & 63;
        for (int e0 = 0; e0 < E; e0 += 8) {
            float acc[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
            for (int64_t k0 = 8 * kl; k0 < a.N; k0 += 512) {
                uint4 xr[4], wr[8];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    xr[i] = (4 * wv + i < nb) ? ld16(a.X + (base + 4 * wv + i) * a.N + k0)
                                              : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int j = 0; j < 8; ++j) wr[j] = ld16(a.Wr + (k0 + j) * E + e0);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const uint32_t ww[4] = {wr[j].x, wr[j].y, wr[j].z, wr[j].w};
                    float wf[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) { wf[2 * q] = bf16_lo(ww[q]); wf[2 * q + 1] = bf16_hi(ww[q]); }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t xw[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
                        const float x = (j & 1) ? bf16_hi(xw[j >> 1]) : bf16_lo(xw[j >> 1]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(x, wf[e], acc[i][e]);
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) s_red[wv][8 * i + e][kl] = acc[i][e];
            __syncthreads();
            if (kl < 32) {
                float sum = 0.f;
                for (int l = 0; l < 64; ++l) sum += s_red[wv][kl][l];
                const int e = e0 + (kl & 7);
                s_log[(4 * wv + (kl >> 3)) * E + e] = sum + (a.br ? a.br[e] : 0.f);
            }
            __syncthreads();
        }
    } else {
        // stage the block's logits with coalesced loads, 8 in flight per thread
        const int n = nb * E;
        const float* src = a.logits + base * E;
        for (int i0 = tid; i0 < n; i0 += 8 * kTopkThreads) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kTopkThreads;
                v[u] = i < n ? src[i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kTopkThreads;
                if (i < n) s_log[i] = v[u];
            }
        }
        __syncthreads();
    }

    if (tid < nb) {
        const int64_t t = base + tid;
        float bv[k];
        int be[k];
        topk_row<k>(s_log + tid * E, E, bv, be);
        float ex[k];
        float den = 0.f;
#pragma unroll
        for (int s = 0; s < k; ++s) {
            ex[s] = expf(bv[s] - bv[0]);
            den += ex[s];
        }
#pragma unroll
        for (int s = 0; s < k; ++s) {
            a.ids[t * k + s] = be[s];
            a.w[t * k + s] = ex[s] / den;
            atomicAdd(&s_cnt[be[s]], 1);   // a count: the order of the adds does not matter
        }
    }
    __syncthreads();
    for (int e = tid; e < E; e += kTopkThreads) a.blk_counts[(int64_t)blockIdx.x * E + e] = s_cnt[e];
    if (kRouter && a.logits_out)
        for (int i = tid; i < nb * E; i += kTopkThreads) a.logits_out[base * E + i] = s_log[i];
}

// Per-expert totals and exclusive offsets, the base position of every
// scatter block in every expert's list, and the tile table (heaviest expert
// first, ties to the smaller index; tiles of at most 64 rows).  One
// workgroup: for each expert, tpe threads each own a contiguous run of
// scatter blocks; integer sums only.
__global__ __launch_bounds__(kScanThreads) void moe_scan_kernel(
    const int32_t* __restrict__ blk_counts, int64_t nblk_a, int group, int64_t nblk_b, int E,
    int32_t* counts, int32_t* offsets, int32_t* blk_base, int32_t* tiles, int32_t* tile_count) {
    __shared__ int s_part[kScanThreads];
    __shared__ int s_tot[kMaxE];
    __shared__ int s_off[kMaxE];
    __shared__ int s_order[kMaxE];
    __shared__ int s_tstart[kMaxE + 1];
    const int tid = threadIdx.x;
    int epow = 1;
    while (epow < E) epow <<= 1;
    const int tpe = kScanThreads / epow;
    const int e = tid / tpe, r = tid % tpe;
    const bool act = e < E;
    const int64_t per = (nblk_b + tpe - 1) / tpe;
    const int64_t b0 = r * per;
    const int64_t b1 = (b0 + per) < nblk_b ? (b0 + per) : nblk_b;
    auto bcount = [&](int64_t bb) {
        int c = 0;
        for (int q = 0; q < group; ++q) {
            const int64_t ba = bb * group + q;
            if (ba < nblk_a) c += blk_counts[ba * E + e];
        }
        return c;
    };
    int sum = 0;
    if (act)
        for (int64_t bb = b0; bb < b1; ++bb) sum += bcount(bb);
    s_part[tid] = sum;
    __syncthreads();
    // only the first nparts threads of an expert own blocks (the rest hold
    // zeros): the prefix and the total loop over those alone (a loop over all
    // tpe = 1024 / E threads cost ~10 us of serial LDS reads at E = 8)
    const int nparts = per > 0 ? (int)((nblk_b + per - 1) / per) : 0;
    int pre = 0;
    if (act) {
        const int upto = r < nparts ? r : nparts;
        for (int q = 0; q < upto; ++q) pre += s_part[e * tpe + q];
        if (r == 0) {
            int tot = 0;
            for (int q = 0; q < nparts; ++q) tot += s_part[e * tpe + q];
            s_tot[e] = tot;
        }
    }
    __syncthreads();
    // one thread per expert: its offset (the totals of the experts before
    // it), its place in the heaviest-first order (ties to the smaller index)
    // and its first tile (the tiles of the experts placed before it); every
    // thread reads all E totals, so no step waits on another's result
    if (tid < E) {
        const int x = tid, tx = s_tot[x];
        int off = 0, place = 0, first = 0, all = 0;
        for (int y = 0; y < E; ++y) {
            const int ty = s_tot[y];
            const int ny = (ty + kBM - 1) / kBM;
            all += ny;
            if (y < x) off += ty;
            if (ty > tx || (ty == tx && y < x)) {
                ++place;
                first += ny;
            }
        }
        s_off[x] = off;
        counts[x] = tx;
        offsets[x] = off;
        s_order[place] = x;
        s_tstart[place] = first;
        if (x == E - 1) offsets[E] = off + tx;
        if (x == 0) {
            s_tstart[E] = all;
            *tile_count = all;
        }
    }
    __syncthreads();
    if (act) {
        int run = s_off[e] + pre;
        for (int64_t bb = b0; bb < b1; ++bb) {
            blk_base[bb * E + e] = run;
            run += bcount(bb);
        }
    }
    const int ntiles = s_tstart[E];
    for (int i = tid; i < ntiles; i += kScanThreads) {
        // the place p with s_tstart[p] <= i < s_tstart[p + 1]: a bisection
        // that keeps s_tstart[lo] <= i < s_tstart[hi] (true at 0 and E)
        int lo = 0, hi = E;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_tstart[mid] <= i) lo = mid;
            else hi = mid;
        }
        const int p = lo;
        const int x = s_order[p];
        const int r0 = (i - s_tstart[p]) * kBM;
        tiles[3 * i + 0] = x;
        tiles[3 * i + 1] = s_off[x] + r0;
        tiles[3 * i + 2] = (s_tot[x] - r0) < kBM ? (s_tot[x] - r0) : kBM;
    }
}

// Stable scatter of the entries t*k+s into their experts' lists, in token
// order, one block of 256 tokens per workgroup: inside a wave each entry is
// ranked among the wave's entries of the same expert with a ballot; one
// barrier publishes the per-wave counts; the position is the block's base
// for the expert plus the counts of earlier waves plus the rank.
template <int k>
__global__ __launch_bounds__(kScatterTokens) void moe_scatter_kernel(
    const int32_t* __restrict__ ids, int64_t M, int E, const int32_t* __restrict__ blk_base,
    int32_t* sorted, int32_t* pos) {
    __shared__ int s_wcnt[kScatterTokens / 64][kMaxE];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t = (int64_t)blockIdx.x * kScatterTokens + tid;
    const bool have = t < M;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int mine[k], rank[k];
#pragma unroll
    for (int s = 0; s < k; ++s) {
        mine[s] = have ? ids[t * k + s] : -1;
        rank[s] = 0;
    }
    for (int e = 0; e < E; ++e) {
        bool hit = false;   // the k picks of a token are distinct experts
#pragma unroll
        for (int s = 0; s < k; ++s) hit |= (mine[s] == e);
        const uint64_t mask = __ballot(hit);
        const int r = __popcll(mask & lt_mask);
#pragma unroll
        for (int s = 0; s < k; ++s)
            if (mine[s] == e) rank[s] = r;
        if (lane == 0) s_wcnt[wave][e] = __popcll(mask);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < k; ++s) {
        const int e = mine[s];
        if (e < 0) continue;
        int before = 0;
        for (int q = 0; q < wave; ++q) before += s_wcnt[q][e];
        const int p = blk_base[(int64_t)blockIdx.x * E + e] + before + rank[s];
        sorted[p] = (int32_t)(t * k + s);
        pos[t * k + s] = p;
    }
}

// Combine: Y[t] = sum over the token's k experts j (ascending) of
// w_j * act2(sum of the split partials of its sorted row (ascending) + b2[e_j]).
__global__ __launch_bounds__(256) void moe_combine_kernel(
    const char* __restrict__ part, int splits, int64_t rows_total, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ ids, const float* __restrict__ w, const uint16_t* __restrict__ b2,
    uint16_t* __restrict__ Y, int64_t M, int k, int64_t P, int act2) {
    const int64_t nvec = M * (P / 8);
    const int64_t split_stride = rows_total * P;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = v / (P / 8);
        const int64_t p = (v - t * (P / 8)) * 8;
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < k; ++j) {
            const int64_t r = pos[t * k + j];
            const int64_t e = ids[t * k + j];
            const float wt = w[t * k + j];
            // packed partials (kPartBytes each), splits summed in ascending order
            const char* src = part + (r * P + p) * kPartBytes;
            float z[8];
            load_f24x8(src, z);
            for (int s = 1; s < splits; ++s) {
                float t[8];
                load_f24x8(src + s * split_stride * kPartBytes, t);
#pragma unroll
                for (int i = 0; i < 8; ++i) z[i] += t[i];
            }
            if (b2) {
                uint4 bb = ld16(b2 + e * P + p);
                uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[2 * i] += bf16_lo(bw[i]);
                    z[2 * i + 1] += bf16_hi(bw[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = fmaf(wt, apply_act(act2, z[i]), y[i]);
        }
        uint4 o = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                             pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
        *reinterpret_cast<uint4*>(Y + t * P + p) = o;
    }
}

// The same combine with the top-k count and the split count fixed at compile
// time: every partial load of a thread is issued before the first is used
// (MoE workload, 4 splits: 80.4 -> 78.9 us; 16 values per thread with 16-byte
// loads measured no faster).  Same summation order, so the same bits.
template <int kK, int kS>
__global__ __launch_bounds__(256) void moe_combine_fixed_kernel(
    const char* __restrict__ part, int64_t rows_total, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ ids, const float* __restrict__ w, const uint16_t* __restrict__ b2,
    uint16_t* __restrict__ Y, int64_t M, int64_t P, int act2) {
    constexpr int kWords = 8 * kPartBytes / 4;   // eight packed values
    const int64_t nvec = M * (P / 8);
    const int64_t split_bytes = rows_total * P * kPartBytes;
    for (int64_t v = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; v < nvec;
         v += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = v / (P / 8);
        const int64_t p = (v - t * (P / 8)) * 8;
        int64_t e[kK];
        float wt[kK];
        uint32_t raw[kK][kS][kWords];
#pragma unroll
        for (int j = 0; j < kK; ++j) {
            const int64_t r = pos[t * kK + j];
            e[j] = ids[t * kK + j];
            wt[j] = w[t * kK + j];
            const char* src = part + (r * P + p) * kPartBytes;
#pragma unroll
            for (int s = 0; s < kS; ++s)
#pragma unroll
                for (int q = 0; q < kWords / 2; ++q) {
                    const uint2 u = *reinterpret_cast<const uint2*>(src + s * split_bytes + 8 * q);
                    raw[j][s][2 * q] = u.x;
                    raw[j][s][2 * q + 1] = u.y;
                }
        }
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kK; ++j) {
            float z[8];
            unpack_f24x4(raw[j][0][0], raw[j][0][1], raw[j][0][2], z);
            unpack_f24x4(raw[j][0][3], raw[j][0][4], raw[j][0][5], z + 4);
#pragma unroll
            for (int s = 1; s < kS; ++s) {
                float u[8];
                unpack_f24x4(raw[j][s][0], raw[j][s][1], raw[j][s][2], u);
                unpack_f24x4(raw[j][s][3], raw[j][s][4], raw[j][s][5], u + 4);
#pragma unroll
                for (int i = 0; i < 8; ++i) z[i] += u[i];
            }
            if (b2) {
                uint4 bb = ld16(b2 + e[j] * P + p);
                uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    z[2 * i] += bf16_lo(bw[i]);
                    z[2 * i + 1] += bf16_hi(bw[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = fmaf(wt[j], apply_act(act2, z[i]), y[i]);
        }
        uint4 o = make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                             pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7]));
        *reinterpret_cast<uint4*>(Y + t * P + p) = o;
    }
}

}  // namespace

int64_t moe_max_tiles(int64_t M, int64_t E, int k) {
    return (M * k + E * (kBM - 1)) / kBM;
}

int64_t moe_route_blocks_a(int64_t M, int64_t E, bool router) {
    const int tb = topk_block_tokens(E, router);
    return (M + tb - 1) / tb;
}

int64_t moe_route_blocks_b(int64_t M) { return (M + kScatterTokens - 1) / kScatterTokens; }

hipError_t launch_moe_route(const RouteIO& io, hipStream_t stream) {
    const bool router = io.logits == nullptr;
    TopkArgs a;
    a.logits = io.logits;
    a.X = io.X;
    a.Wr = io.Wr;
    a.br = io.br;
    a.logits_out = io.logits_out;
    a.M = io.M;
    a.N = io.N;
    a.E = (int)io.E;
    a.tb = topk_block_tokens(io.E, router);
    a.ids = io.ids;
    a.w = io.w;
    a.blk_counts = io.blk_counts;
    const int64_t na = moe_route_blocks_a(io.M, io.E, router);
    const int64_t nbk = moe_route_blocks_b(io.M);
    if (na <= 0) return hipSuccess;
    switch (io.k) {
#define FFN_TOPK_K(K)                                                                             \
    case K:                                                                                       \
        if (router)                                                                               \
            hipLaunchKernelGGL((moe_topk_kernel<K, true>), dim3((unsigned)na), dim3(kTopkThreads), \
                               0, stream, a);                                                     \
        else                                                                                      \
            hipLaunchKernelGGL((moe_topk_kernel<K, false>), dim3((unsigned)na),                   \
                               dim3(kTopkThreads), 0, stream, a);                                 \
        break;
        FFN_TOPK_K(1) FFN_TOPK_K(2) FFN_TOPK_K(3) FFN_TOPK_K(4)
        FFN_TOPK_K(5) FFN_TOPK_K(6) FFN_TOPK_K(7) FFN_TOPK_K(8)
#undef FFN_TOPK_K
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, io.blk_counts, na,
                       kScatterTokens / a.tb, nbk, a.E, io.counts, io.offsets, io.blk_base,
                       io.tiles, io.tile_count);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (io.k) {
#define FFN_SCATTER_K(K)                                                                        \
    case K:                                                                                     \
        hipLaunchKernelGGL(moe_scatter_kernel<K>, dim3((unsigned)nbk), dim3(kScatterTokens), 0, \
                           stream, io.ids, io.M, a.E, io.blk_base, io.sorted, io.pos);          \
        break;
        FFN_SCATTER_K(1) FFN_SCATTER_K(2) FFN_SCATTER_K(3) FFN_SCATTER_K(4)
        FFN_SCATTER_K(5) FFN_SCATTER_K(6) FFN_SCATTER_K(7) FFN_SCATTER_K(8)
#undef FFN_SCATTER_K
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_moe_combine(const void* part, int splits, int64_t rows_total,
                              const int32_t* pos, const int32_t* ids, const float* w,
                              const uint16_t* b2, uint16_t* Y, int64_t M, int k, int64_t P,
                              int act2, hipStream_t stream) {
    const int64_t nvec = M * (P / 8);
    if (nvec <= 0) return hipSuccess;
    int64_t blocks = (nvec + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    const char* pp = static_cast<const char*>(part);
#define FFN_COMBINE_FIXED(K, S)                                                              \
    if (k == K && splits == S) {                                                             \
        hipLaunchKernelGGL((moe_combine_fixed_kernel<K, S>), dim3((unsigned)blocks), dim3(256), \
                           0, stream, pp, rows_total, pos, ids, w, b2, Y, M, P, act2);       \
        return hipGetLastError();                                                            \
    }
    FFN_COMBINE_FIXED(1, 1) FFN_COMBINE_FIXED(1, 2) FFN_COMBINE_FIXED(1, 4) FFN_COMBINE_FIXED(1, 8)
    FFN_COMBINE_FIXED(2, 1) FFN_COMBINE_FIXED(2, 2) FFN_COMBINE_FIXED(2, 4) FFN_COMBINE_FIXED(2, 8)
#undef FFN_COMBINE_FIXED
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, pp, splits,
                       rows_total, pos, ids, w, b2, Y, M, k, P, act2);
    return hipGetLastError();
}

}  // namespace ffn
