/*
 * Host sanitizer run of the CPU oracle (test infrastructure): built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
 * together with oracle/hsq_oracle.c, it calls every oracle entry point on
 * small seeded inputs (group 64 and 128, rank 0 and 4, row subsets, windows
 * at the matrix edges) and checks a few invariants; any out-of-bounds
 * access, use of uninitialised heap or undefined arithmetic aborts the run.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float oracle_bf16_to_f32(uint16_t b);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_f16_rne(float x);
void oracle_quantize_act_g(const uint16_t *X, int M, int K, int group, const uint16_t *lam, int8_t *q,
                           uint16_t *sx, float *xh);
void oracle_pack_act(const int8_t *q, int M, int K, uint8_t *packed);
void oracle_group_partials_g(const int8_t *qa, const int8_t *qw, int M, int K, int N, int group, int m0,
                             int mc, int n0, int nc, int32_t *P);
void oracle_lowrank_down(const float *xh, int M, int K, const uint16_t *L1, int r, double *U);
void oracle_linear_g(const uint16_t *X, int M, int K, int N, int group, const uint16_t *lam, const int8_t *qw,
                     const uint16_t *sw, const uint16_t *L1, const uint16_t *L2, int r, const uint16_t *bias,
                     const int *rows, int nrows, double *Y);

static uint32_t state = 12345u;
static uint32_t next(void) {          /* xorshift32: seeded test data only */
    state ^= state << 13;
    state ^= state >> 17;
    state ^= state << 5;
    return state;
}
static uint16_t bf16_of(float f) {    /* truncation is fine for test inputs */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}
static float uniform(void) { return (float)(next() & 0xFFFFFF) / 16777216.0f * 2.0f - 1.0f; }

static int run(int M, int K, int N, int r, int group) {
    int G = K / group;
    uint16_t *X = malloc(sizeof(uint16_t) * M * K), *lam = malloc(sizeof(uint16_t) * K);
    uint16_t *sw = malloc(sizeof(uint16_t) * G * N), *L1 = malloc(sizeof(uint16_t) * K * (r ? r : 1));
    uint16_t *L2 = malloc(sizeof(uint16_t) * (r ? r : 1) * N), *bias = malloc(sizeof(uint16_t) * N);
    int8_t *qw = malloc((size_t)K * N), *q = malloc((size_t)M * K);
    uint16_t *sx = malloc(sizeof(uint16_t) * M * G);
    float *xh = malloc(sizeof(float) * M * K);
    uint8_t *packed = malloc((size_t)M * K / 2);
    int32_t *P = malloc(sizeof(int32_t) * M * N * G);
    double *U = malloc(sizeof(double) * M * (r ? r : 1)), *Y = malloc(sizeof(double) * (M > 3 ? M : 3) * N);
    int rows[3] = {0, M / 2, M - 1};
    for (int i = 0; i < M * K; ++i) X[i] = bf16_of(uniform() * (i % 97 == 0 ? 30.0f : 1.0f));
    for (int m = 0; m < M; m += 5)                         /* zero groups */
        for (int k = 0; k < group; ++k) X[m * K + k] = 0;
    for (int k = 0; k < K; ++k) lam[k] = oracle_f32_to_f16_rne(0.5f + (float)(next() % 1000) / 700.0f);
    for (int i = 0; i < G * N; ++i) sw[i] = oracle_f32_to_f16_rne(1e-3f + (float)(next() % 1000) * 1e-5f);
    for (int i = 0; i < K * N; ++i) qw[i] = (int8_t)((int)(next() % 16) - 8);
    for (int i = 0; i < K * (r ? r : 1); ++i) L1[i] = bf16_of(uniform() * 0.02f);
    for (int i = 0; i < (r ? r : 1) * N; ++i) L2[i] = bf16_of(uniform() * 0.02f);
    for (int i = 0; i < N; ++i) bias[i] = bf16_of(uniform() * 0.02f);

    oracle_quantize_act_g(X, M, K, group, lam, q, sx, xh);
    for (int i = 0; i < M * K; ++i)
        if (q[i] < -8 || q[i] > 7) return fprintf(stderr, "code out of range\n"), 1;
    oracle_pack_act(q, M, K, packed);
    oracle_group_partials_g(q, qw, M, K, N, group, 0, M, 0, N, P);
    oracle_group_partials_g(q, qw, M, K, N, group, M - 1, 1, N - 1, 1, P);   /* corner window */
    if (r) oracle_lowrank_down(xh, M, K, L1, r, U);
    oracle_linear_g(X, M, K, N, group, lam, qw, sw, r ? L1 : NULL, r ? L2 : NULL, r, bias, NULL, M, Y);
    oracle_linear_g(X, M, K, N, group, lam, qw, sw, r ? L1 : NULL, r ? L2 : NULL, r, NULL, rows, 3, Y);
    (void)oracle_bf16_to_f32(X[0]);
    (void)oracle_f16_to_f32(sx[0]);
    free(X); free(lam); free(sw); free(L1); free(L2); free(bias); free(qw); free(q); free(sx);
    free(xh); free(packed); free(P); free(U); free(Y);
    return 0;
}

int main(void) {
    /* every fp16 pattern through both conversions */
    for (uint32_t h = 0; h < 65536; ++h) {
        float f = oracle_f16_to_f32((uint16_t)h);
        if (f == f && oracle_f32_to_f16_rne(f) != (uint16_t)h && (h & 0x7FFF) != 0)
            return fprintf(stderr, "fp16 round trip %x\n", h), 1;
    }
    int fails = 0;
    fails += run(19, 256, 37, 4, 64);
    fails += run(19, 256, 37, 0, 128);
    fails += run(33, 384, 20, 5, 64);
    fails += run(1, 128, 1, 1, 128);
    if (fails) return 1;
    printf("oracle sanitizer run ok\n");
    return 0;
}
