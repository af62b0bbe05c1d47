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

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxE = 256;
constexpr int kLogitStage = 8192;   // floats of router logits staged in LDS per token block

// One workgroup.  Pass 1 stages a block of router logits in LDS with coalesced
// loads and gives each token to one thread (top-k by insertion into a list
// sorted by decreasing logit, an equal logit staying behind the earlier
// expert, which is the repeated strict arg-max order), then the gate weights
// and the expert histogram.  Pass 2 scatters the entries into the per-expert
// lists in token order: inside a block every wave ranks its entries per
// expert with ballots, one barrier publishes the per-wave counts, and each
// entry's position is the expert's running offset plus the counts of earlier
// waves plus its rank.
template <int k>
__global__ __launch_bounds__(kRouteThreads) void moe_route_kernel(
    const float* __restrict__ logits, int64_t M, int E, int32_t* ids, float* w,
    int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* pos, int32_t* tiles,
    int32_t* tile_count) {
    __shared__ float s_log[kLogitStage];
    __shared__ int s_cnt[kMaxE];
    __shared__ int s_run[kMaxE];
    __shared__ int s_off[kMaxE];
    __shared__ int s_wcnt[kRouteWaves][kMaxE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    for (int e = tid; e < E; e += kRouteThreads) s_cnt[e] = 0;

    // ---- pass 1: top-k and gate weights per token, expert histogram
    const int tb = (kLogitStage / E) < kRouteThreads ? (kLogitStage / E) : kRouteThreads;
    for (int64_t base = 0; base < M; base += tb) {
        const int nb = (M - base) < tb ? (int)(M - base) : tb;
        __syncthreads();   // the previous block's logits are no longer read
        for (int i0 = tid; i0 < nb * E; i0 += 8 * kRouteThreads) {   // 8 loads in flight
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kRouteThreads;
                v[u] = i < nb * E ? logits[base * E + i] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kRouteThreads;
                if (i < nb * E) s_log[i] = v[u];
            }
        }
        __syncthreads();
        const bool act = tid < nb;
        const int64_t t = base + tid;
        const float* row = s_log + tid * E;
        float bv[k];
        int be[k];
#pragma unroll
        for (int j = 0; j < k; ++j) { bv[j] = 0.f; be[j] = 0; }
        int nf = 0;
        for (int e = 0; act && e < E; ++e) {
            const float v = row[e];
            int p = 0;   // entries that stay ahead: larger or equal logit
#pragma unroll
            for (int j = 0; j < k; ++j) p += (j < nf && bv[j] >= v) ? 1 : 0;
            if (p >= k) continue;
#pragma unroll
            for (int j = k - 1; j > 0; --j)
                if (j > p && j < k) { bv[j] = bv[j - 1]; be[j] = be[j - 1]; }
#pragma unroll
            for (int j = 0; j < k; ++j)
                if (j == p) { bv[j] = v; be[j] = e; }
            nf = nf + 1 < k ? nf + 1 : k;
        }
        float ex[k];
        float den = 0.f;
#pragma unroll
        for (int s = 0; s < k; ++s) {
            if (s < k) {
                ex[s] = expf(bv[s] - bv[0]);
                den += ex[s];
            }
        }
#pragma unroll
        for (int s = 0; s < k; ++s) {
            if (act && s < k) {
                ids[t * k + s] = be[s];
                w[t * k + s] = ex[s] / den;
            }
        }
        // expert histogram: one LDS add per wave and expert (ballot counts), not
        // one contended add per entry
        for (int e = 0; e < E; ++e) {
            int c = 0;
#pragma unroll
            for (int s = 0; s < k; ++s) c += __popcll(__ballot(act && s < k && be[s] == e));
            if (lane == 0 && c) atomicAdd(&s_cnt[e], c);
        }
    }
    __syncthreads();

    // ---- per-expert counts and exclusive offsets
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < E; ++e) {
            counts[e] = s_cnt[e];
            offsets[e] = run;
            s_run[e] = run;
            s_off[e] = run;
            run += s_cnt[e];
        }
        offsets[E] = run;
    }
    __syncthreads();

    // ---- pass 2: stable scatter, entry t*k+s into its expert's list in token order
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t base = 0; base < M; base += kRouteThreads) {
        const int64_t t = base + tid;
        const bool have = t < M;
        int mine[k], rank[k];
#pragma unroll
        for (int s = 0; s < k; ++s) {
            mine[s] = (have && s < k) ? ids[t * k + s] : -1;
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
            const int p = s_run[e] + before + rank[s];
            sorted[p] = (int32_t)(t * k + s);
            pos[t * k + s] = p;
        }
        __syncthreads();
        for (int e = tid; e < E; e += kRouteThreads) {
            int tot = 0;
            for (int q = 0; q < kRouteWaves; ++q) tot += s_wcnt[q][e];
            s_run[e] += tot;
        }
        __syncthreads();
    }

    // ---- tile table, heaviest expert first (ties: smaller index first)
    if (tid == 0) {
        int n = 0;
        int* done = &s_wcnt[0][0];   // the per-wave counts are no longer needed
        for (int e = 0; e < E; ++e) done[e] = 0;
        for (int it = 0; it < E; ++it) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!done[e] && (best < 0 || s_cnt[e] > s_cnt[best])) best = e;
            done[best] = 1;
            for (int r0 = 0; r0 < s_cnt[best]; r0 += kBM) {
                const int v = (s_cnt[best] - r0) < kBM ? (s_cnt[best] - r0) : kBM;
                tiles[3 * n + 0] = best;
                tiles[3 * n + 1] = s_off[best] + r0;
                tiles[3 * n + 2] = v;
                ++n;
            }
        }
        *tile_count = n;
    }
}

__global__ __launch_bounds__(256) void moe_combine_kernel(
    const float* __restrict__ part, int splits, int64_t rows_total, const int32_t* __restrict__ pos,
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
            const float* src = part + r * P + p;
            float4 lo = *reinterpret_cast<const float4*>(src);
            float4 hi = *reinterpret_cast<const float4*>(src + 4);
            float z[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
            for (int s = 1; s < splits; ++s) {
                const float* q = src + s * split_stride;
                lo = *reinterpret_cast<const float4*>(q);
                hi = *reinterpret_cast<const float4*>(q + 4);
                z[0] += lo.x; z[1] += lo.y; z[2] += lo.z; z[3] += lo.w;
                z[4] += hi.x; z[5] += hi.y; z[6] += hi.z; z[7] += hi.w;
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

}  // namespace

int64_t moe_max_tiles(int64_t M, int64_t E, int k) {
    return (M * k + E * (kBM - 1)) / kBM;
}

hipError_t launch_moe_route(const float* logits, int64_t M, int64_t E, int k, int32_t* ids,
                            float* w, int32_t* counts, int32_t* offsets, int32_t* sorted,
                            int32_t* pos, int32_t* tiles, int32_t* tile_count,
                            hipStream_t stream) {
    switch (k) {
#define FFN_ROUTE_K(K)                                                                          \
    case K:                                                                                      \
        hipLaunchKernelGGL(moe_route_kernel<K>, dim3(1), dim3(kRouteThreads), 0, stream, logits, \
                           M, (int)E, ids, w, counts, offsets, sorted, pos, tiles, tile_count);  \
        break;
        FFN_ROUTE_K(1) FFN_ROUTE_K(2) FFN_ROUTE_K(3) FFN_ROUTE_K(4)
        FFN_ROUTE_K(5) FFN_ROUTE_K(6) FFN_ROUTE_K(7) FFN_ROUTE_K(8)
#undef FFN_ROUTE_K
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_moe_combine(const float* part, int splits, int64_t rows_total,
                              const int32_t* pos, const int32_t* ids, const float* w,
                              const uint16_t* b2, uint16_t* Y, int64_t M, int k, int64_t P,
                              int act2, hipStream_t stream) {
    const int64_t nvec = M * (P / 8);
    if (nvec <= 0) return hipSuccess;
    int64_t blocks = (nvec + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part,
                       splits, rows_total, pos, ids, w, b2, Y, M, k, P, act2);
    return hipGetLastError();
}

}  // namespace ffn
