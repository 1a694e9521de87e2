/*
 * hsq_oracle.c -- the plain, slow CPU oracle for the W4A4 + rank-r linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant with the
 * HIP library; the two meet only through the seeded input generator.
 *
 * What it computes (cited to the pages; the method is an encoding, so the
 * quantizer follows the steps in order, and the contraction is the plain
 * definition written out):
 *
 *   Deflating the Hessian (abstract): each weight is split into a low-bit
 *   residual and a high-precision low-rank component, W ~ L1*L2 + Q(R).
 *   Deflating the Hessian (Table 1 caption; Table 8 caption): 4-bit weights
 *   and 4-bit activations, group-64 for the diffusion transformers;
 *   (Table 3, 4, 6 and 7 captions): group-128 for the Qwen3-8B runs.  The
 *   group width is a parameter (64 or 128) of the functions ending in _g;
 *   the others are their group-64 forms.
 *   H-SVDQuant explainer (rit.work), section on Hessian deflation, last
 *   paragraph: a diagonal scaling moves range between weights and
 *   activations and leaves the full-precision transform unchanged.
 *   DiRotQ notes (papernotes.org), key design 2: the two-branch inference
 *   form runs its high-precision branch on unquantized activations.
 *
 * Arithmetic contract (the pages print no inference formula; these are the
 * readings this library states and both sides follow):
 *   xh[m,k]  = fl32( float(X[m,k]) * fl32(1 / float(lambda[k])) )
 *   amax     = max over the group (64 or 128 channels) of |xh|
 *   s        = 0 if amax == 0, else f16_rne( fl32(amax / 7) ), saturated at 65504
 *   q[m,k]   = 0 if s == 0, else clamp( rint( fl32(xh * fl32(1 / float(s))) ), -8, 7 )
 *   P[m,n,g] = sum_{k in g} q[m,k] * qw[k,n]                   (exact integer)
 *   Y[m,n]   = sum_g P*s[m,g]*sw[g,n] + sum_j U[m,j]*L2[j,n] + b[n]   (fp64)
 *   U[m,j]   = sum_k xh[m,k] * L1[k,j]                                  (fp64)
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared -ffp-contract=off (no fast-math).
 * On x86-64 float arithmetic is IEEE binary32 (SSE), so every fl32 above is
 * a single correctly rounded operation.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_GROUP 64          /* the default group width */
#define ORACLE_MAX_GROUP 128

/* ---- number formats, written from the IEEE-754 / bfloat16 definitions ---- */

/* bfloat16 is the top half of a binary32 word: the conversion is exact. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);    /* (1.f) * 2^(e-15) */
    return (float)(sign ? -v : v);                /* exact: fits binary32 */
}

/* binary32 -> binary16, round to nearest, ties to even.  The representable
 * binary16 values near |x| are multiples of a quantum: 2^-24 below the
 * smallest normal 2^-14, else 2^(e-10) for |x| in [2^e, 2^(e+1)).  The
 * scaled value |x|/quantum is exact in double; rint() (default rounding
 * mode, ties to even) picks the nearest multiple.  A carry out of the
 * fraction lands in the exponent field by plain addition. */
uint16_t oracle_f32_to_f16_rne(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0;
    double a = fabs((double)x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0)                 /* halfway to 2^16 and beyond: inf */
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        double n = rint(ldexp(a, 24));            /* multiples of 2^-24 */
        return (uint16_t)(sign | (uint16_t)n);    /* n == 1024 -> 2^-14 */
    }
    int E;
    frexp(a, &E);                                 /* a = f * 2^E, f in [0.5,1) */
    int e = E - 1;                                /* a in [2^e, 2^(e+1)) */
    double n = rint(ldexp(a, 10 - e));            /* in [1024, 2048] */
    unsigned bits = ((unsigned)(e + 15) << 10) + (unsigned)(n - 1024.0);
    if (bits >= 0x7c00u)
        bits = 0x7c00u;
    return (uint16_t)(sign | bits);
}

/* ---- step 1-4: smoothing and per-token group-wise symmetric int4 codes ---- */

/* Quantize rows [0, M) of X (M x K bf16, row-major) in groups of `group`
 * consecutive channels (64 or 128).
 *   lam  : K fp16 smoothing factors (x is divided by lambda, via its
 *          fp32 reciprocal).
 *   q    : M x K int8 codes out.
 *   sx   : M x (K/group) fp16 scales out.
 *   xh   : optional M x K fp32 smoothed activations out (NULL to skip).
 * K must be a multiple of group; inputs must be finite. */
void oracle_quantize_act_g(const uint16_t *X, int M, int K, int group, const uint16_t *lam,
                           int8_t *q, uint16_t *sx, float *xh)
{
    int G = K / group;
    float *inv_lam = (float *)malloc(sizeof(float) * (size_t)K);
    for (int k = 0; k < K; ++k)
        inv_lam[k] = 1.0f / oracle_f16_to_f32(lam[k]);

#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        float v[ORACLE_MAX_GROUP];
        for (int g = 0; g < G; ++g) {
            size_t base = (size_t)m * K + (size_t)g * group;
            float amax = 0.0f;
            for (int j = 0; j < group; ++j) {
                int k = g * group + j;
                v[j] = oracle_bf16_to_f32(X[base + j]) * inv_lam[k];
                if (fabsf(v[j]) > amax)
                    amax = fabsf(v[j]);
                if (xh)
                    xh[base + j] = v[j];
            }
            uint16_t s16 = 0;
            if (amax != 0.0f) {
                s16 = oracle_f32_to_f16_rne(amax / 7.0f);
                if (s16 == 0x7c00u)
                    s16 = 0x7bffu;                    /* saturate at 65504 */
            }
            sx[(size_t)m * G + g] = s16;
            if (s16 == 0) {
                for (int j = 0; j < group; ++j)
                    q[base + j] = 0;
                continue;
            }
            float inv_s = 1.0f / oracle_f16_to_f32(s16);
            for (int j = 0; j < group; ++j) {
                float t = v[j] * inv_s;
                float r = rintf(t);                   /* ties to even */
                int c = r > 7.0f ? 7 : (r < -8.0f ? -8 : (int)r);
                q[base + j] = (int8_t)c;
            }
        }
    }
    free(inv_lam);
}

void oracle_quantize_act(const uint16_t *X, int M, int K, const uint16_t *lam,
                         int8_t *q, uint16_t *sx, float *xh)
{
    oracle_quantize_act_g(X, M, K, ORACLE_GROUP, lam, q, sx, xh);
}

/* Canonical packed activation layout: byte j of a row holds code k = 2j in
 * its low nibble and k = 2j+1 in its high nibble, two's complement. */
void oracle_pack_act(const int8_t *q, int M, int K, uint8_t *packed)
{
    for (int m = 0; m < M; ++m)
        for (int j = 0; j < K / 2; ++j) {
            uint8_t lo = (uint8_t)q[(size_t)m * K + 2 * j] & 0x0f;
            uint8_t hi = (uint8_t)q[(size_t)m * K + 2 * j + 1] & 0x0f;
            packed[(size_t)m * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

/* ---- step 5: per-group integer partial sums, brute force ---- */

/* P[(m-m0)][(n-n0)][g] = sum_{k in group g} qa[m,k] * qw[k,n], groups of
 * `group` channels; qa: M x K int8 (row-major), qw: K x N int8 (row-major,
 * in x out). */
void oracle_group_partials_g(const int8_t *qa, const int8_t *qw, int M, int K, int N, int group,
                             int m0, int mc, int n0, int nc, int32_t *P)
{
    int G = K / group;
    (void)M;
#pragma omp parallel for schedule(static)
    for (int i = 0; i < mc; ++i) {
        int m = m0 + i;
        for (int jn = 0; jn < nc; ++jn) {
            int n = n0 + jn;
            for (int g = 0; g < G; ++g) {
                int32_t acc = 0;
                for (int t = 0; t < group; ++t) {
                    int k = g * group + t;
                    acc += (int32_t)qa[(size_t)m * K + k] * (int32_t)qw[(size_t)k * N + n];
                }
                P[((size_t)i * nc + jn) * G + g] = acc;
            }
        }
    }
}

void oracle_group_partials(const int8_t *qa, const int8_t *qw, int M, int K, int N,
                           int m0, int mc, int n0, int nc, int32_t *P)
{
    oracle_group_partials_g(qa, qw, M, K, N, ORACLE_GROUP, m0, mc, n0, nc, P);
}

/* ---- step 4b: the rank-r down projection on the smoothed, unquantized x ---- */

/* U[m][j] = sum_k xh[m,k] * L1[k,j]  in fp64; L1 is K x r bf16 row-major. */
void oracle_lowrank_down(const float *xh, int M, int K, const uint16_t *L1, int r,
                         double *U)
{
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m)
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k)
                acc += (double)xh[(size_t)m * K + k] *
                       (double)oracle_bf16_to_f32(L1[(size_t)k * r + j]);
            U[(size_t)m * r + j] = acc;
        }
}

/* ---- steps 1-7 together, for a chosen set of output rows ---- */

/* Y[i][n] for rows m = rows[i] (rows == NULL: all M rows, i == m), fp64,
 * with groups of `group` channels (64 or 128).
 *   X (M x K bf16), lam (K fp16), qw (K x N int8 codes), sw ((K/group) x N fp16),
 *   L1 (K x r bf16), L2 (r x N bf16), bias (N bf16 or NULL); r may be 0.
 * Each chosen row is quantized on its own (rows are independent: the
 * quantizer is per token), then every (n, g) partial is a brute-force
 * integer dot product. */
void oracle_linear_g(const uint16_t *X, int M, int K, int N, int group, const uint16_t *lam,
                     const int8_t *qw, const uint16_t *sw, const uint16_t *L1,
                     const uint16_t *L2, int r, const uint16_t *bias,
                     const int *rows, int nrows, double *Y)
{
    int G = K / group;
    int count = rows ? nrows : M;
#pragma omp parallel
    {
        int8_t *q = (int8_t *)malloc((size_t)K);
        uint16_t *s = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)G);
        float *xh = (float *)malloc(sizeof(float) * (size_t)K);
        double *u = (double *)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < count; ++i) {
            int m = rows ? rows[i] : i;
            oracle_quantize_act_g(X + (size_t)m * K, 1, K, group, lam, q, s, xh);
            if (r > 0)
                oracle_lowrank_down(xh, 1, K, L1, r, u);
            for (int n = 0; n < N; ++n) {
                double y = 0.0;
                for (int g = 0; g < G; ++g) {
                    int32_t p = 0;
                    for (int t = 0; t < group; ++t) {
                        int k = g * group + t;
                        p += (int32_t)q[k] * (int32_t)qw[(size_t)k * N + n];
                    }
                    y += (double)p * (double)oracle_f16_to_f32(s[g]) *
                         (double)oracle_f16_to_f32(sw[(size_t)g * N + n]);
                }
                for (int j = 0; j < r; ++j)
                    y += u[j] * (double)oracle_bf16_to_f32(L2[(size_t)j * N + n]);
                if (bias)
                    y += (double)oracle_bf16_to_f32(bias[n]);
                Y[(size_t)i * N + n] = y;
            }
        }
        free(q);
        free(s);
        free(xh);
        free(u);
    }
}

void oracle_linear(const uint16_t *X, int M, int K, int N, const uint16_t *lam,
                   const int8_t *qw, const uint16_t *sw, const uint16_t *L1,
                   const uint16_t *L2, int r, const uint16_t *bias,
                   const int *rows, int nrows, double *Y)
{
    oracle_linear_g(X, M, K, N, ORACLE_GROUP, lam, qw, sw, L1, L2, r, bias, rows, nrows, Y);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
