/*
 * Host-sanitizer driver for the C oracle (oracle/recursive.c), built with
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers.py
 * and run on the CPU: ragged shapes, every leaf size class, per-row and
 * per-group grids, tie following, and the argument errors.  Exits non-zero
 * when a run disagrees with itself across leaf sizes (Theorem 3.2: every
 * split gives the same rounding) or an argument error is not reported; the
 * sanitizers abort on any memory or undefined-behaviour fault.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_bakron_recursive_grouped(int64_t m, int64_t n, const double* W, const double* PA, const double* PB,
                                    const float* s, const float* z, const int32_t* maxq, int64_t group, int64_t gld,
                                    int64_t leaf, int32_t* codes, double* V, double* E, const int32_t* follow,
                                    double tau, int64_t* adoptions);
int oracle_bakron_recursive(int64_t m, int64_t n, const double* W, const double* PA, const double* PB,
                            const float* s, const float* z, const int32_t* maxq, int64_t leaf, int32_t* codes,
                            double* V, double* E);

static uint64_t rng = 88172645463325252ull;
static double urand(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

/* unit lower triangular with small random entries below the diagonal */
static double* unit_lower(int64_t n)
{
    double* P = calloc((size_t)(n * n), sizeof(double));
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t j = 0; j < i; ++j) P[i * n + j] = 0.3 * (urand() - 0.5) / (double)(1 + i - j);
        P[i * n + i] = 1.0;
    }
    return P;
}

static int run(int64_t m, int64_t n, int64_t group)
{
    const int64_t gld = group >= n ? 1 : (n + group - 1) / group;
    const int64_t ng = m * gld;
    double* W = malloc(sizeof(double) * (size_t)(m * n));
    for (int64_t k = 0; k < m * n; ++k) W[k] = urand() - 0.5;
    double* PA = unit_lower(n);
    double* PB = unit_lower(m);
    float* s = malloc(sizeof(float) * (size_t)ng);
    float* z = malloc(sizeof(float) * (size_t)ng);
    int32_t* q = malloc(sizeof(int32_t) * (size_t)ng);
    for (int64_t k = 0; k < ng; ++k) {
        s[k] = (float)(0.1 + 0.2 * urand());
        z[k] = (float)(3.0 * urand());
        q[k] = 1 + (int32_t)(7 * urand());
    }
    int32_t* c1 = malloc(sizeof(int32_t) * (size_t)(m * n));
    int32_t* c2 = malloc(sizeof(int32_t) * (size_t)(m * n));
    double* V = malloc(sizeof(double) * (size_t)(m * n));
    double* E = malloc(sizeof(double) * (size_t)(m * n));
    int bad = 0;
    int64_t adopt = -1;
    if (oracle_bakron_recursive_grouped(m, n, W, PA, PB, s, z, q, group, gld, 1, c1, V, E, NULL, 0.0, &adopt) != 0)
        bad = 1;
    const int64_t leaves[3] = {2, 5, 32};
    for (int l = 0; l < 3 && !bad; ++l) {
        if (oracle_bakron_recursive_grouped(m, n, W, PA, PB, s, z, q, group, gld, leaves[l], c2, V, E, NULL, 0.0,
                                            NULL) != 0 ||
            memcmp(c1, c2, sizeof(int32_t) * (size_t)(m * n)) != 0)
            bad = 2;
    }
    /* following its own codes adopts nothing */
    if (!bad && (oracle_bakron_recursive_grouped(m, n, W, PA, PB, s, z, q, group, gld, 7, c2, V, E, c1, 0.5,
                                                 &adopt) != 0 ||
                 adopt != 0 || memcmp(c1, c2, sizeof(int32_t) * (size_t)(m * n)) != 0))
        bad = 3;
    if (!bad && gld == 1 && (oracle_bakron_recursive(m, n, W, PA, PB, s, z, q, 16, c2, V, E) != 0 ||
                             memcmp(c1, c2, sizeof(int32_t) * (size_t)(m * n)) != 0))
        bad = 4;
    printf("oracle %lldx%lld group %lld: %s\n", (long long)m, (long long)n, (long long)group, bad ? "FAIL" : "ok");
    free(W); free(PA); free(PB); free(s); free(z); free(q); free(c1); free(c2); free(V); free(E);
    return bad;
}

int main(void)
{
    int bad = 0;
    const int64_t shapes[][3] = {{1, 1, 1}, {1, 9, 9}, {9, 1, 1}, {7, 11, 3}, {33, 17, 17}, {40, 70, 32},
                                 {65, 64, 64}, {100, 37, 8}, {129, 131, 131}};
    for (size_t k = 0; k < sizeof(shapes) / sizeof(shapes[0]); ++k)
        bad |= run(shapes[k][0], shapes[k][1], shapes[k][2]);
    /* argument errors */
    double d = 0.0;
    float f = 1.0f;
    int32_t i = 1;
    int64_t a = 0;
    if (oracle_bakron_recursive_grouped(-1, 2, &d, &d, &d, &f, &f, &i, 1, 1, 1, &i, &d, &d, NULL, 0.0, &a) != -1 ||
        oracle_bakron_recursive_grouped(2, 2, &d, &d, &d, &f, &f, &i, 1, 1, 0, &i, &d, &d, NULL, 0.0, &a) != -1 ||
        oracle_bakron_recursive_grouped(2, 4, &d, &d, &d, &f, &f, &i, 2, 1, 1, &i, &d, &d, NULL, 0.0, &a) != -1 ||
        oracle_bakron_recursive_grouped(2, 2, NULL, &d, &d, &f, &f, &i, 2, 1, 1, &i, &d, &d, NULL, 0.0, &a) != -1 ||
        oracle_bakron_recursive_grouped(0, 5, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 1, NULL, NULL, NULL, NULL,
                                        0.0, &a) != 0) {
        printf("argument errors: FAIL\n");
        bad |= 8;
    }
    printf(bad ? "ORACLE SANITIZE FAIL\n" : "ORACLE SANITIZE OK\n");
    return bad;
}
