/* Exercises every entry point of oracle/oracle.c on small inputs, for the
 * AddressSanitizer / UndefinedBehaviorSanitizer build run by
 * tests/test_sanitizers.py.  Exits non-zero if any call reports an error;
 * the sanitizers abort on the first invalid access or undefined operation. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_ffn(int, const void*, const void*, const void*, const void*, const void*,
               const int64_t*, int64_t, int64_t, int64_t, int64_t, int64_t, int, int, double*);
int oracle_swiglu(int, const void*, const void*, const void*, const void*, const int64_t*,
                  int64_t, int64_t, int64_t, int64_t, int64_t, double*);
int oracle_ffn_backward(int, const void*, const void*, const void*, const void*, const void*,
                        int64_t, int64_t, int64_t, int64_t, int, const int64_t*, int64_t, double*,
                        const int64_t*, int64_t, double*, double*, double*, double*);
int oracle_router_logits(int, const void*, const void*, const float*, const int64_t*, int64_t,
                         int64_t, int64_t, int64_t, double*);
int oracle_moe_route(const float*, int64_t, int64_t, int, int32_t*, double*, int32_t*, int32_t*,
                     int32_t*);
int oracle_moe_ffn(int, const void*, const float*, int64_t, int64_t, int, const void*, const void*,
                   const void*, const void*, int64_t, int64_t, int64_t, int, int, const int64_t*,
                   int64_t, double*);
double oracle_act(int, double);
double oracle_act_grad(int, double);

static uint32_t state = 12345u;
static float rnd(void) {   /* uniform in [-1, 1) from a 32-bit LCG */
    state = state * 1664525u + 1013904223u;
    return (float)((double)(state >> 8) / (double)(1u << 23) - 1.0);
}
static float* farr(size_t n) {
    float* p = (float*)malloc(n * sizeof(float));
    for (size_t i = 0; i < n; ++i) p[i] = rnd();
    return p;
}
static uint16_t* barr(size_t n) {   /* bf16 patterns: the upper half of an fp32 draw */
    uint16_t* p = (uint16_t*)malloc(n * sizeof(uint16_t));
    for (size_t i = 0; i < n; ++i) {
        float f = rnd();
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        p[i] = (uint16_t)(u >> 16);
    }
    return p;
}

#define CHECK(call)                                              \
    do {                                                         \
        if ((call) != 0) {                                       \
            fprintf(stderr, "failed: %s (line %d)\n", #call, __LINE__); \
            return 1;                                            \
        }                                                        \
    } while (0)

int main(void) {
    const int64_t M = 5, N = 24, O = 40, P = 16, E = 4;
    const int k = 2;
    for (int dt = 0; dt < 2; ++dt) {   /* fp32, then bf16 */
        void *X, *W1, *b1, *W2, *b2, *Wu, *dY, *Wr;
        if (dt == 0) {
            X = farr(M * N); W1 = farr(N * O); b1 = farr(O); W2 = farr(O * P); b2 = farr(P);
            Wu = farr(N * O); dY = farr(M * P); Wr = farr(N * E);
        } else {
            X = barr(M * N); W1 = barr(N * O); b1 = barr(O); W2 = barr(O * P); b2 = barr(P);
            Wu = barr(N * O); dY = barr(M * P); Wr = barr(N * E);
        }
        double* Y = (double*)malloc(M * P * sizeof(double));
        const int64_t rows[3] = {4, 0, 2};
        for (int act = 0; act < 3; ++act) {
            CHECK(oracle_ffn(dt, X, W1, b1, W2, b2, NULL, 0, M, N, O, P, act, act, Y));
            CHECK(oracle_ffn(dt, X, W1, NULL, W2, NULL, rows, 3, M, N, O, P, act, 0, Y));
        }
        CHECK(oracle_swiglu(dt, X, W1, Wu, W2, NULL, 0, M, N, O, P, Y));
        CHECK(oracle_swiglu(dt, X, W1, Wu, W2, rows, 3, M, N, O, P, Y));
        double* dX = (double*)malloc(M * N * sizeof(double));
        double* dW1 = (double*)malloc(N * O * sizeof(double));
        double* db1 = (double*)malloc(O * sizeof(double));
        double* dW2 = (double*)malloc(O * P * sizeof(double));
        double* db2 = (double*)malloc(P * sizeof(double));
        const int64_t cols[2] = {39, 3};
        for (int act = 0; act < 3; ++act) {
            CHECK(oracle_ffn_backward(dt, X, W1, b1, W2, dY, M, N, O, P, act, NULL, 0, dX, NULL, 0,
                                      dW1, db1, dW2, db2));
            CHECK(oracle_ffn_backward(dt, X, W1, NULL, W2, dY, M, N, O, P, act, rows, 3, dX, cols, 2,
                                      dW1, db1, dW2, db2));
        }
        float br[4] = {0.8f, 0.4f, -0.2f, -0.8f};
        double* lgd = (double*)malloc(M * E * sizeof(double));
        CHECK(oracle_router_logits(dt, X, Wr, br, NULL, 0, M, N, E, lgd));
        CHECK(oracle_router_logits(dt, X, Wr, NULL, rows, 3, M, N, E, lgd));
        float* lg = (float*)malloc(M * E * sizeof(float));
        for (int64_t i = 0; i < M * E; ++i) lg[i] = (float)lgd[i];
        int32_t ids[10], counts[4], offsets[5], sorted[10];
        double w[10];
        CHECK(oracle_moe_route(lg, M, E, k, ids, w, counts, offsets, sorted));
        void *EW1, *Eb1, *EW2, *Eb2;
        if (dt == 0) { EW1 = farr(E * N * O); Eb1 = farr(E * O); EW2 = farr(E * O * P); Eb2 = farr(E * P); }
        else { EW1 = barr(E * N * O); Eb1 = barr(E * O); EW2 = barr(E * O * P); Eb2 = barr(E * P); }
        CHECK(oracle_moe_ffn(dt, X, lg, M, E, k, EW1, Eb1, EW2, Eb2, N, O, P, 2, 0, NULL, 0, Y));
        CHECK(oracle_moe_ffn(dt, X, lg, M, E, k, EW1, NULL, EW2, NULL, N, O, P, 1, 2, rows, 3, Y));
        /* rejected arguments return -1 without touching memory */
        if (oracle_ffn(dt, NULL, W1, b1, W2, b2, NULL, 0, M, N, O, P, 1, 0, Y) != -1) return 2;
        if (oracle_moe_route(lg, M, E, 5, ids, w, counts, offsets, sorted) != -1) return 2;
        free(X); free(W1); free(b1); free(W2); free(b2); free(Wu); free(dY); free(Wr); free(Y);
        free(dX); free(dW1); free(db1); free(dW2); free(db2); free(lgd); free(lg);
        free(EW1); free(Eb1); free(EW2); free(Eb2);
    }
    for (double x = -12.0; x <= 12.0; x += 0.25) {
        (void)oracle_act(2, x);
        (void)oracle_act_grad(2, x);
    }
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
