/*
 * Sequential BaKron-recursive in float64 -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests, the smoke check and the bench CPU baseline may load this
 * library.  It shares no code with the HIP solver.
 *
 * What it computes (pages cited by title):
 *   [S] paper summary "FastKron: Efficient Quantization with
 *       Kronecker-Factored Hessians", derivation naive -> antidiagonal ->
 *       BaKron and Theorem 3.2.
 * The rounding of W (m x n) under the Hessian A (x) B, in a divide-and-conquer
 * order: a block is split into quadrants Q11, Q12, Q21, Q22 (or halves when
 * one side is already small); Q11 is solved first, its raw errors are pushed
 * into Q12, Q21 and Q22 by dense products PB[rows', rows] E PA[cols', cols]^T,
 * then Q12 is solved and pushed into Q22, then Q21 is solved and pushed into
 * Q22, then Q22 is solved.  Any such order visits an entry after all entries
 * above and to the left of it, so by Theorem 3.2 it gives the output of
 * BaKron-naive.  The pages name a recursive variant without defining its
 * split; this quadtree is the reading taken here.  Leaves of at most
 * `leaf` x `leaf` entries run the naive rule: quantize one entry, then
 * W~[i', j'] -= e * PB[i', i] * PA[j', j] over the leaf's bottom-right part.
 *
 * Base quantizer (uniform grid per output row, or per (row, group of `group`
 * input columns): entry (i, j) uses grid entry i * gld + j / group, so a
 * per-row grid is group >= n, gld = 1; the grids are fixed inputs): the decision
 * x = float32(float32(w) / s) + z is taken in float32 arithmetic, the code is
 * clamp(rint(x), 0, maxq) (round half to even), the value is s (c - z) in
 * float64, and the raw error is e = w~ - value.
 *
 * Tie-following mode (for comparing against another implementation): given
 * that implementation's codes `follow`, at an entry whose float32 decision x
 * lies within `tau` grid steps of a rounding boundary (x = k + 1/2) and whose
 * followed code is the neighbouring one (one step away), the oracle takes the
 * followed code and counts an adoption.  Near such a boundary float32 and
 * float64 arithmetic may legitimately round either way (Theorem 3.2's
 * equality is exact only in exact arithmetic), and one flip changes every
 * later entry below and to the right; following keeps the two trajectories
 * together so that every other decision can be compared exactly.  Elsewhere
 * the oracle keeps its own decision.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared.  OpenMP only
 * splits the rows of the dense propagation products; the summation order of
 * each dot product is fixed by `omp simd` lanes, so results may differ from a
 * serial build by float64 rounding only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t m, n, leaf;
    const double* PA;   /* n x n, unit lower triangular, row-major */
    const double* PB;   /* m x m, unit lower triangular, row-major */
    const float* s;
    const float* z;
    const int32_t* maxq;
    int64_t group, gld;  /* grid of entry (i, j): index i * gld + j / group */
    double* Wt;         /* m x n working weights */
    double* E;          /* m x n raw errors */
    int32_t* codes;     /* m x n */
    double* V;          /* m x n */
    double* T;          /* scratch: rows x cols of the largest pushed block */
    const int32_t* follow;   /* NULL, or codes to follow at near-ties */
    double tau;
    int64_t adoptions;
} ctx_t;

/* Returns the float32 decision x; sets the code and value. */
static float quant(double w, float s, float z, int32_t maxq, int32_t* code, double* val)
{
    float wf = (float)w;
    float x = wf / s;
    x = x + z;
    float c = rintf(x);
    if (c < 0.0f) c = 0.0f;
    if (c > (float)maxq) c = (float)maxq;
    *code = (int32_t)c;
    *val = (double)s * ((double)c - (double)z);
    return x;
}

/* Distance (in grid steps) of x from the nearest rounding boundary k + 1/2
 * with 0 <= k < maxq (beyond them the clamp decides). */
static double margin_of(float x, int32_t maxq)
{
    double b = floor((double)x) + 0.5;
    if (b < 0.5) b = 0.5;
    if (b > (double)maxq - 0.5) b = (double)maxq - 0.5;
    return fabs((double)x - b);
}

/* Naive rule on rows [r0,r1) x cols [c0,c1), column-major visiting order. */
static void leaf_solve(ctx_t* X, int64_t r0, int64_t r1, int64_t c0, int64_t c1)
{
    const int64_t n = X->n, m = X->m;
    int64_t nc = c1 - c0;
    /* local transposed copy of PA[c0:c1, c0:c1] so the update loop is unit stride */
    double* pat = (double*)malloc(sizeof(double) * (size_t)(nc * nc));
    for (int64_t a = 0; a < nc; ++a)
        for (int64_t b = 0; b < nc; ++b)
            pat[a * nc + b] = X->PA[(c0 + b) * n + (c0 + a)];   /* pat[j][j'] = PA[j'][j] */
    for (int64_t j = c0; j < c1; ++j) {
        for (int64_t i = r0; i < r1; ++i) {
            int32_t c;
            double v;
            double w = X->Wt[i * n + j];
            const int64_t gi = i * X->gld + j / X->group;
            const float x = quant(w, X->s[gi], X->z[gi], X->maxq[gi], &c, &v);
            if (X->follow) {
                const int32_t g = X->follow[i * n + j];
                if ((g == c + 1 || g == c - 1) && margin_of(x, X->maxq[gi]) < X->tau) {
                    c = g;
                    v = (double)X->s[gi] * ((double)c - (double)X->z[gi]);
                    X->adoptions += 1;
                }
            }
            double e = w - v;
            X->codes[i * n + j] = c;
            X->V[i * n + j] = v;
            X->E[i * n + j] = e;
            const double* prow = pat + (j - c0) * nc;
            for (int64_t ii = i; ii < r1; ++ii) {
                double f = e * X->PB[ii * m + i];
                double* wr = X->Wt + ii * n;
                for (int64_t jj = j; jj < c1; ++jj)
                    wr[jj] -= f * prow[jj - c0];
            }
        }
    }
    free(pat);
}

/*
 * Push the raw errors of source block S = [sr0,sr1) x [sc0,sc1) into target
 * block [tr0,tr1) x [tc0,tc1), which lies below and/or right of S:
 *   Wt[t] -= PB[trows, srows] * E[S] * PA[tcols, scols]^T
 * First T = E[S] * PA[tcols, scols]^T (|srows| x |tcols|), then the left
 * product.  Rows of each product are split over OpenMP threads.
 */
static void push(ctx_t* X, int64_t sr0, int64_t sr1, int64_t sc0, int64_t sc1,
                 int64_t tr0, int64_t tr1, int64_t tc0, int64_t tc1)
{
    const int64_t n = X->n, m = X->m;
    const int64_t R = sr1 - sr0, Cc = tc1 - tc0, K = sc1 - sc0;
    double* T = X->T;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        const double* er = X->E + (sr0 + r) * n + sc0;
        for (int64_t u = 0; u < Cc; ++u) {
            const double* pr = X->PA + (tc0 + u) * n + sc0;
            double acc = 0.0;
            #pragma omp simd reduction(+:acc)
            for (int64_t k = 0; k < K; ++k) acc += er[k] * pr[k];
            T[r * Cc + u] = acc;
        }
    }
    #pragma omp parallel for schedule(static)
    for (int64_t t = tr0; t < tr1; ++t) {
        double* wr = X->Wt + t * n + tc0;
        const double* pb = X->PB + t * m;
        for (int64_t r = 0; r < R; ++r) {
            double f = pb[sr0 + r];
            if (f == 0.0) continue;
            const double* tr = T + r * Cc;
            #pragma omp simd
            for (int64_t u = 0; u < Cc; ++u) wr[u] -= f * tr[u];
        }
    }
}

static void solve_block(ctx_t* X, int64_t r0, int64_t r1, int64_t c0, int64_t c1)
{
    int64_t R = r1 - r0, C = c1 - c0;
    if (R <= 0 || C <= 0) return;
    if (R <= X->leaf && C <= X->leaf) {
        leaf_solve(X, r0, r1, c0, c1);
        return;
    }
    if (R > X->leaf && C > X->leaf) {
        int64_t rm = r0 + R / 2, cm = c0 + C / 2;
        solve_block(X, r0, rm, c0, cm);                               /* Q11 */
        push(X, r0, rm, c0, cm, r0, rm, cm, c1);                      /* -> Q12 */
        push(X, r0, rm, c0, cm, rm, r1, c0, c1);                      /* -> Q21, Q22 */
        solve_block(X, r0, rm, cm, c1);                               /* Q12 */
        push(X, r0, rm, cm, c1, rm, r1, cm, c1);                      /* -> Q22 */
        solve_block(X, rm, r1, c0, cm);                               /* Q21 */
        push(X, rm, r1, c0, cm, rm, r1, cm, c1);                      /* -> Q22 */
        solve_block(X, rm, r1, cm, c1);                               /* Q22 */
    } else if (R > X->leaf) {
        int64_t rm = r0 + R / 2;
        solve_block(X, r0, rm, c0, c1);
        push(X, r0, rm, c0, c1, rm, r1, c0, c1);
        solve_block(X, rm, r1, c0, c1);
    } else {
        int64_t cm = c0 + C / 2;
        solve_block(X, r0, r1, c0, cm);
        push(X, r0, r1, c0, cm, r0, r1, cm, c1);
        solve_block(X, r0, r1, cm, c1);
    }
}

/*
 * Returns 0 on success, -1 on bad arguments, -2 on allocation failure.
 * W, PA, PB: float64 row-major; s, z: float32 grid; maxq: int32; entry
 * (i, j) uses grid entry i * gld + j / group (per row: group >= n, gld = 1;
 * per group of g columns: group = g, gld = ceil(n / g)).
 * Outputs codes (int32), V and E (float64), all m x n row-major.
 * follow (nullable, m x n int32) and tau select the tie-following mode;
 * *adoptions (nullable) receives the number of codes taken over.
 */
int oracle_bakron_recursive_grouped(int64_t m, int64_t n, const double* W, const double* PA,
                                    const double* PB, const float* s, const float* z,
                                    const int32_t* maxq, int64_t group, int64_t gld, int64_t leaf,
                                    int32_t* codes, double* V, double* E, const int32_t* follow,
                                    double tau, int64_t* adoptions)
{
    if (adoptions) *adoptions = 0;
    if (m < 0 || n < 0 || leaf < 1 || group < 1 || gld < 1) return -1;
    if (m == 0 || n == 0) return 0;
    if (!W || !PA || !PB || !s || !z || !maxq || !codes || !V || !E) return -1;
    if ((n - 1) / group >= gld) return -1;   /* the last column's group must exist */
    ctx_t X;
    X.m = m; X.n = n; X.leaf = leaf;
    X.PA = PA; X.PB = PB; X.s = s; X.z = z; X.maxq = maxq;
    X.group = group; X.gld = gld;
    X.codes = codes; X.V = V; X.E = E;
    X.follow = follow; X.tau = tau; X.adoptions = 0;
    X.Wt = (double*)malloc(sizeof(double) * (size_t)(m * n));
    /* largest pushed block: half the rows times all the columns */
    X.T = (double*)malloc(sizeof(double) * (size_t)(((m + 1) / 2 + leaf) * n + 1));
    if (!X.Wt || !X.T) { free(X.Wt); free(X.T); return -2; }
    memcpy(X.Wt, W, sizeof(double) * (size_t)(m * n));
    memset(E, 0, sizeof(double) * (size_t)(m * n));
    solve_block(&X, 0, m, 0, n);
    free(X.Wt);
    free(X.T);
    if (adoptions) *adoptions = X.adoptions;
    return 0;
}

/* Per-row grids (s, z, maxq of length m). */
int oracle_bakron_recursive_follow(int64_t m, int64_t n, const double* W, const double* PA,
                                   const double* PB, const float* s, const float* z,
                                   const int32_t* maxq, int64_t leaf, int32_t* codes,
                                   double* V, double* E, const int32_t* follow, double tau,
                                   int64_t* adoptions)
{
    return oracle_bakron_recursive_grouped(m, n, W, PA, PB, s, z, maxq, n > 0 ? n : 1, 1, leaf, codes, V, E,
                                           follow, tau, adoptions);
}

int oracle_bakron_recursive(int64_t m, int64_t n, const double* W, const double* PA,
                            const double* PB, const float* s, const float* z,
                            const int32_t* maxq, int64_t leaf, int32_t* codes,
                            double* V, double* E)
{
    return oracle_bakron_recursive_follow(m, n, W, PA, PB, s, z, maxq, leaf, codes, V, E, NULL, 0.0, NULL);
}
