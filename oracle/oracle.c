/*
 * oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation, in fp64, of what the
 * fused feed-forward path computes.  Only the test suite, the package smoke
 * check and the benchmark's CPU-baseline leg may load or call this library.
 * The product path never does: it shares no code, header, table or helper
 * with the HIP kernels, and the HIP side never calls into it.
 *
 * Sources (cited by page title and section; no code appears on the pages):
 *  - the kernel-fusion / tensor-parallelism post (brunomaga.github.io),
 *    section "Megatron-LM tensor parallelism", the equations for H and Y:
 *    H = act(X W1 + b1), Y = act2(H W2 + b2), X: MxN, W1: NxO, b1: O,
 *    W2: OxP, b2: P; the second activation is optional.
 *  - Same page, same section, the tensor-parallel equation: the per-shard
 *    partial H^(g) W2^(g) carries no b2; b2 (and act2) are applied once after
 *    the sum over shards.  oracle_ffn() with b2 == NULL computes that partial.
 *  - Same post, section "Benchmarks": a SwiGLU FFN has a third weight matrix
 *    whose product with the input gates the activation, and no biases.
 *    oracle_swiglu() computes H = silu(X Wg) * (X Wu) elementwise and
 *    Y = H Wd, with silu(x) = x / (1 + exp(-x)) (the Swish-1 / SiLU unit of
 *    Ramachandran et al. and Elfwing et al.; the page names the activation
 *    but does not write it out).
 *  - Same post, closing section: a fused backward pass is named as the next
 *    step.  oracle_ffn_backward() is the plain chain rule of the two layers
 *    (act2 none): with a = X W1 + b1, h = act1(a), Y = h W2 + b2 and the
 *    output gradient dY: dh = dY W2^T, da = dh * act1'(a), dX = da W1^T,
 *    dW1 = X^T da, db1 = sum_m da, dW2 = h^T dY, db2 = sum_m dY.
 *  - "Fine-Grained Compute-Communication Overlap for MoE" review
 *    (zhongzhuzhou.org), section 2.1 (Mixture-of-Experts, briefly) and 2.2
 *    (five steps): the router picks the top-k experts per token and the
 *    output is the gate-weighted sum of those experts' FFN outputs.
 *    Step 1 runs "the gate" (a small router network) on the tokens;
 *    oracle_router_logits() reads it as one linear layer, the plainest form
 *    (as in Switch Transformer and GShard, which the section names):
 *    logits = X Wr + br.
 *
 * Readings where the pages are silent:
 *  - act1 is ReLU or the tanh form of GELU; GELU-tanh is
 *    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) (Hendrycks & Gimpel).
 *  - top-k ties go to the smaller expert index; slot 0 holds the largest logit.
 *  - gate weights are a softmax over the k selected logits only.
 *  - per-expert token lists hold entries t*k+s in ascending t.
 *
 * Everything is computed in double from the exact input values (bf16 bits are
 * widened exactly; fp32 is widened exactly).  Nothing is rounded to bf16.
 * Each sum runs in ascending index order; the bias is added after the sum.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_ACT_NONE = 0, OR_ACT_RELU = 1, OR_ACT_GELU_TANH = 2 };

/* Threads the OpenMP loops below use (reported with the CPU baseline). */
int oracle_threads(void) { return omp_get_max_threads(); }

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load(int dtype, const void* base, int64_t idx) {
    if (dtype == OR_BF16) return bf16_bits_to_double(((const uint16_t*)base)[idx]);
    return (double)((const float*)base)[idx];
}

double oracle_act(int act, double x) {
    if (act == OR_ACT_RELU) return x > 0.0 ? x : 0.0;
    if (act == OR_ACT_GELU_TANH) {
        const double c = sqrt(2.0 / M_PI);
        return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
    }
    return x;
}

/* Derivative of act1: ReLU' = 1 for x > 0, else 0 (0 at the kink); GELU-tanh'
 * = 0.5 (1 + tanh u) + 0.5 x (1 - tanh^2 u) u'(x), u = sqrt(2/pi) (x + 0.044715 x^3),
 * u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2); none: 1. */
double oracle_act_grad(int act, double x) {
    if (act == OR_ACT_RELU) return x > 0.0 ? 1.0 : 0.0;
    if (act == OR_ACT_GELU_TANH) {
        const double c = sqrt(2.0 / M_PI);
        const double t = tanh(c * (x + 0.044715 * x * x * x));
        return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * c * (1.0 + 3.0 * 0.044715 * x * x);
    }
    return 1.0;
}

/* One output row of the two-layer FFN, straight from the definition.
 * h[o] = act1( sum_n X[m,n] W1[n,o]  + b1[o] )
 * y[p] = act2( sum_o h[o]   W2[o,p]  + b2[p] )
 * Work arrays h (O) and acc (max(O,P)) are supplied by the caller. */
static void ffn_row(int dtype, const void* X, const void* W1, const void* b1,
                    const void* W2, const void* b2, int64_t m, int64_t N,
                    int64_t O, int64_t P, int act1, int act2,
                    double* h, double* acc, double* yrow) {
    /* layer 1: each acc[o] accumulates over n in ascending order */
    for (int64_t o = 0; o < O; ++o) acc[o] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double x = load(dtype, X, m * N + n);
        for (int64_t o = 0; o < O; ++o) acc[o] += x * load(dtype, W1, n * O + o);
    }
    for (int64_t o = 0; o < O; ++o) {
        double a = acc[o] + (b1 ? load(dtype, b1, o) : 0.0);
        h[o] = oracle_act(act1, a);
    }
    /* layer 2: each acc[p] accumulates over o in ascending order */
    for (int64_t p = 0; p < P; ++p) acc[p] = 0.0;
    for (int64_t o = 0; o < O; ++o) {
        double hv = h[o];
        for (int64_t p = 0; p < P; ++p) acc[p] += hv * load(dtype, W2, o * P + p);
    }
    for (int64_t p = 0; p < P; ++p) {
        double a = acc[p] + (b2 ? load(dtype, b2, p) : 0.0);
        yrow[p] = oracle_act(act2, a);
    }
}

/* Y[r, :] for r in rows[0..nrows) (all M rows when rows == NULL, nrows = M).
 * Y is nrows x P doubles.  b1/b2 may be NULL (zero bias): b2 == NULL with
 * act2 == NONE gives one tensor-parallel shard's partial output.
 * Returns 0, or -1 on bad arguments. */
int oracle_ffn(int dtype, const void* X, const void* W1, const void* b1,
               const void* W2, const void* b2, const int64_t* rows, int64_t nrows,
               int64_t M, int64_t N, int64_t O, int64_t P, int act1, int act2,
               double* Y) {
    if (!X || !W1 || !W2 || !Y || M < 0 || N < 1 || O < 1 || P < 1) return -1;
    if (dtype != OR_F32 && dtype != OR_BF16) return -1;
    if (!rows) nrows = M;
    int bad = 0;
#pragma omp parallel
    {
        int64_t wn = O > P ? O : P;
        double* h = (double*)malloc(sizeof(double) * (size_t)O);
        double* acc = (double*)malloc(sizeof(double) * (size_t)wn);
        if (!h || !acc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t m = rows ? rows[r] : r;
                if (m < 0 || m >= M) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                ffn_row(dtype, X, W1, b1, W2, b2, m, N, O, P, act1, act2, h, acc,
                        Y + r * P);
            }
        }
        free(h);
        free(acc);
    }
    return bad ? -1 : 0;
}

/* silu(x) = x * sigmoid(x), written as x / (1 + exp(-x)). */
double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* One output row of the SwiGLU FFN:
 * g[o] = sum_n X[m,n] Wg[n,o], u[o] = sum_n X[m,n] Wu[n,o]  (ascending n)
 * h[o] = silu(g[o]) * u[o]
 * y[p] = sum_o h[o] Wd[o,p]  (ascending o).  No biases. */
static void swiglu_row(int dtype, const void* X, const void* Wg, const void* Wu,
                       const void* Wd, int64_t m, int64_t N, int64_t O, int64_t P,
                       double* g, double* u, double* acc, double* yrow) {
    for (int64_t o = 0; o < O; ++o) g[o] = u[o] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double x = load(dtype, X, m * N + n);
        for (int64_t o = 0; o < O; ++o) {
            g[o] += x * load(dtype, Wg, n * O + o);
            u[o] += x * load(dtype, Wu, n * O + o);
        }
    }
    for (int64_t o = 0; o < O; ++o) g[o] = oracle_silu(g[o]) * u[o];
    for (int64_t p = 0; p < P; ++p) acc[p] = 0.0;
    for (int64_t o = 0; o < O; ++o) {
        double hv = g[o];
        for (int64_t p = 0; p < P; ++p) acc[p] += hv * load(dtype, Wd, o * P + p);
    }
    for (int64_t p = 0; p < P; ++p) yrow[p] = acc[p];
}

/* SwiGLU FFN rows, as oracle_ffn (rows == NULL: all M rows). */
int oracle_swiglu(int dtype, const void* X, const void* Wg, const void* Wu, const void* Wd,
                  const int64_t* rows, int64_t nrows, int64_t M, int64_t N, int64_t O,
                  int64_t P, double* Y) {
    if (!X || !Wg || !Wu || !Wd || !Y || M < 0 || N < 1 || O < 1 || P < 1) return -1;
    if (dtype != OR_F32 && dtype != OR_BF16) return -1;
    if (!rows) nrows = M;
    int bad = 0;
#pragma omp parallel
    {
        double* g = (double*)malloc(sizeof(double) * (size_t)O);
        double* u = (double*)malloc(sizeof(double) * (size_t)O);
        double* acc = (double*)malloc(sizeof(double) * (size_t)P);
        if (!g || !u || !acc) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t m = rows ? rows[r] : r;
                if (m < 0 || m >= M) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                swiglu_row(dtype, X, Wg, Wu, Wd, m, N, O, P, g, u, acc, Y + r * P);
            }
        }
        free(g);
        free(u);
        free(acc);
    }
    return bad ? -1 : 0;
}

/* a[m][o] (pre-activation, with b1) and dh[m][o] = sum_p dY[m][p] W2[o][p]
 * for one row m and one hidden column o. */
static double bwd_a(int dtype, const void* X, const void* W1, const void* b1, int64_t m,
                    int64_t o, int64_t N, int64_t O) {
    double acc = 0.0;
    for (int64_t n = 0; n < N; ++n) acc += load(dtype, X, m * N + n) * load(dtype, W1, n * O + o);
    return acc + (b1 ? load(dtype, b1, o) : 0.0);
}
static double bwd_dh(int dtype, const void* W2, const void* dY, int64_t m, int64_t o, int64_t P) {
    double acc = 0.0;
    for (int64_t p = 0; p < P; ++p) acc += load(dtype, dY, m * P + p) * load(dtype, W2, o * P + p);
    return acc;
}

/* Gradients of the two-layer FFN (act2 none) for the output gradient dY (M x P).
 * dX for the nrows listed rows (rows == NULL: all M; dX nrows x N); for the
 * ncols listed hidden columns (cols == NULL: all O) dW1 (N x ncols, column c
 * for hidden column cols[c]), db1 (ncols) and dW2 (ncols x P); db2 (P).
 * Any output may be NULL.  Sums run in ascending index order. */
int oracle_ffn_backward(int dtype, const void* X, const void* W1, const void* b1, const void* W2,
                        const void* dY, int64_t M, int64_t N, int64_t O, int64_t P, int act1,
                        const int64_t* rows, int64_t nrows, double* dX, const int64_t* cols,
                        int64_t ncols, double* dW1, double* db1, double* dW2, double* db2) {
    if (!X || !W1 || !W2 || !dY || M < 0 || N < 1 || O < 1 || P < 1) return -1;
    if (dtype != OR_F32 && dtype != OR_BF16) return -1;
    if (act1 < OR_ACT_NONE || act1 > OR_ACT_GELU_TANH) return -1;
    if (!rows) nrows = M;
    if (!cols) ncols = O;
    int bad = 0;
    if (dX) {
#pragma omp parallel
        {
            double* da = (double*)malloc(sizeof(double) * (size_t)O);
            if (!da) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t r = 0; r < nrows; ++r) {
                    const int64_t m = rows ? rows[r] : r;
                    if (m < 0 || m >= M) {
#pragma omp atomic write
                        bad = 1;
                        continue;
                    }
                    for (int64_t o = 0; o < O; ++o)
                        da[o] = bwd_dh(dtype, W2, dY, m, o, P) *
                                oracle_act_grad(act1, bwd_a(dtype, X, W1, b1, m, o, N, O));
                    for (int64_t n = 0; n < N; ++n) {
                        double acc = 0.0;
                        for (int64_t o = 0; o < O; ++o) acc += da[o] * load(dtype, W1, n * O + o);
                        dX[r * N + n] = acc;
                    }
                }
            }
            free(da);
        }
    }
    if (dW1 || db1 || dW2) {
#pragma omp parallel
        {
            double* da = (double*)malloc(sizeof(double) * (size_t)(M + 1));
            double* h = (double*)malloc(sizeof(double) * (size_t)(M + 1));
            if (!da || !h) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t c = 0; c < ncols; ++c) {
                    const int64_t o = cols ? cols[c] : c;
                    if (o < 0 || o >= O) {
#pragma omp atomic write
                        bad = 1;
                        continue;
                    }
                    for (int64_t m = 0; m < M; ++m) {
                        const double a = bwd_a(dtype, X, W1, b1, m, o, N, O);
                        h[m] = oracle_act(act1, a);
                        da[m] = bwd_dh(dtype, W2, dY, m, o, P) * oracle_act_grad(act1, a);
                    }
                    if (dW1)
                        for (int64_t n = 0; n < N; ++n) {
                            double acc = 0.0;
                            for (int64_t m = 0; m < M; ++m) acc += load(dtype, X, m * N + n) * da[m];
                            dW1[n * ncols + c] = acc;
                        }
                    if (db1) {
                        double acc = 0.0;
                        for (int64_t m = 0; m < M; ++m) acc += da[m];
                        db1[c] = acc;
                    }
                    if (dW2)
                        for (int64_t p = 0; p < P; ++p) {
                            double acc = 0.0;
                            for (int64_t m = 0; m < M; ++m) acc += h[m] * load(dtype, dY, m * P + p);
                            dW2[c * P + p] = acc;
                        }
                }
            }
            free(da);
            free(h);
        }
    }
    if (db2)
        for (int64_t p = 0; p < P; ++p) {
            double acc = 0.0;
            for (int64_t m = 0; m < M; ++m) acc += load(dtype, dY, m * P + p);
            db2[p] = acc;
        }
    return bad ? -1 : 0;
}

/* Router logits (the gate network read as one linear layer):
 * logits[t][e] = sum_n X[t][n] Wr[n][e] (ascending n) + br[e].
 * X: M x N and Wr: N x E in `dtype`; br: E floats or NULL.  rows == NULL: all
 * M tokens, else the nrows listed tokens; out is nrows x E doubles. */
int oracle_router_logits(int dtype, const void* X, const void* Wr, const float* br,
                         const int64_t* rows, int64_t nrows, int64_t M, int64_t N, int64_t E,
                         double* out) {
    if (!X || !Wr || !out || M < 0 || N < 1 || E < 1) return -1;
    if (dtype != OR_F32 && dtype != OR_BF16) return -1;
    if (!rows) nrows = M;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t t = rows ? rows[r] : r;
        if (t < 0 || t >= M) {
#pragma omp atomic write
            bad = 1;
            continue;
        }
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n)
                acc += load(dtype, X, t * N + n) * load(dtype, Wr, n * E + e);
            out[r * E + e] = acc + (br ? (double)br[e] : 0.0);
        }
    }
    return bad ? -1 : 0;
}

/* Top-k routing from fp32 gate logits (M x E).
 * ids[t*k+s]: s-th largest logit's expert (ties -> smaller index).
 * w[t*k+s]  : softmax over the k selected logits, in fp64.
 * counts[e], offsets[e] (exclusive prefix sum, offsets[E] = M*k),
 * sorted[offsets[e] + j]: the j-th entry t*k+s routed to e, ascending t.
 * Any output pointer may be NULL except ids and w. */
int oracle_moe_route(const float* logits, int64_t M, int64_t E, int k,
                     int32_t* ids, double* w, int32_t* counts, int32_t* offsets,
                     int32_t* sorted) {
    if (!logits || !ids || !w || M < 0 || E < 1 || k < 1 || k > E) return -1;
    for (int64_t t = 0; t < M; ++t) {
        const float* l = logits + t * E;
        for (int s = 0; s < k; ++s) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int q = 0; q < s; ++q) taken |= (ids[t * k + q] == e);
                if (taken) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: first max wins */
            }
            ids[t * k + s] = (int32_t)best;
        }
        double l0 = (double)l[ids[t * k]];
        double denom = 0.0;
        for (int s = 0; s < k; ++s) denom += exp((double)l[ids[t * k + s]] - l0);
        for (int s = 0; s < k; ++s) w[t * k + s] = exp((double)l[ids[t * k + s]] - l0) / denom;
    }
    if (counts || offsets || sorted) {
        int32_t* cnt = (int32_t*)calloc((size_t)E, sizeof(int32_t));
        if (!cnt) return -1;
        for (int64_t i = 0; i < M * k; ++i) cnt[ids[i]]++;
        int32_t run = 0;
        for (int64_t e = 0; e < E; ++e) {
            if (counts) counts[e] = cnt[e];
            if (offsets) offsets[e] = run;
            if (sorted) {
                int32_t pos = run;
                for (int64_t t = 0; t < M; ++t)
                    for (int s = 0; s < k; ++s)
                        if (ids[t * k + s] == e) sorted[pos++] = (int32_t)(t * k + s);
            }
            run += cnt[e];
        }
        if (offsets) offsets[E] = run;
        free(cnt);
    }
    return 0;
}

/* Mixture-of-Experts layer output for tokens rows[0..nrows) (all when NULL):
 * Y[r] = sum_s w[t,s] * FFN_{ids[t,s]}(X[t]), each expert with its own
 * W1_e (NxO), b1_e (O), W2_e (OxP), b2_e (P); experts stacked along the
 * leading axis.  Y is nrows x P doubles. */
int oracle_moe_ffn(int dtype, const void* X, const float* logits, int64_t M,
                   int64_t E, int k, const void* W1, const void* b1,
                   const void* W2, const void* b2, int64_t N, int64_t O,
                   int64_t P, int act1, int act2, const int64_t* rows,
                   int64_t nrows, double* Y) {
    if (!X || !logits || !W1 || !W2 || !Y || M < 0 || E < 1 || k < 1 || k > E ||
        N < 1 || O < 1 || P < 1)
        return -1;
    if (dtype != OR_F32 && dtype != OR_BF16) return -1;
    if (!rows) nrows = M;
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(M * k + 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(M * k + 1));
    if (!ids || !w) { free(ids); free(w); return -1; }
    if (oracle_moe_route(logits, M, E, k, ids, w, NULL, NULL, NULL)) {
        free(ids); free(w); return -1;
    }
    size_t esz = dtype == OR_BF16 ? 2 : 4;
    int bad = 0;
#pragma omp parallel
    {
        int64_t wn = O > P ? O : P;
        double* h = (double*)malloc(sizeof(double) * (size_t)O);
        double* acc = (double*)malloc(sizeof(double) * (size_t)wn);
        double* z = (double*)malloc(sizeof(double) * (size_t)P);
        if (!h || !acc || !z) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t t = rows ? rows[r] : r;
                if (t < 0 || t >= M) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                double* y = Y + r * P;
                for (int64_t p = 0; p < P; ++p) y[p] = 0.0;
                for (int s = 0; s < k; ++s) {
                    int64_t e = ids[t * k + s];
                    const char* w1 = (const char*)W1 + (size_t)(e * N * O) * esz;
                    const char* w2 = (const char*)W2 + (size_t)(e * O * P) * esz;
                    const char* bb1 = b1 ? (const char*)b1 + (size_t)(e * O) * esz : NULL;
                    const char* bb2 = b2 ? (const char*)b2 + (size_t)(e * P) * esz : NULL;
                    ffn_row(dtype, X, w1, bb1, w2, bb2, t, N, O, P, act1, act2, h, acc, z);
                    for (int64_t p = 0; p < P; ++p) y[p] += w[t * k + s] * z[p];
                }
            }
        }
        free(h);
        free(acc);
        free(z);
    }
    free(ids);
    free(w);
    return bad ? -1 : 0;
}
