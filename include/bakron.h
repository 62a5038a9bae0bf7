/*
 * bakron.h -- C ABI of libbakron.so, the BaKron solver for MI355X (gfx950).
 *
 * BaKron rounds a weight matrix W (m x n) onto a per-output-row uniform grid
 * by GPTQ-style adaptive rounding under a two-sided Kronecker-factored
 * Hessian A (x) B: A (n x n) describes the input side, B (m x m) the output
 * side.  Pages cited by title:
 *   [S] paper summary "FastKron: Efficient Quantization with
 *       Kronecker-Factored Hessians" (arXiv 2608.06291): setup, derivation
 *       naive -> antidiagonal -> BaKron, Proposition 3.1, Theorem 3.2,
 *       Corollary 3.4;
 *   [A] paper page "BaKron: Efficient Quantization with Kronecker-Factored
 *       Hessians": abstract (O(m+n) sequential steps, O(mn(m+n)) work,
 *       modular base quantizer).
 *
 * Conventions for every entry point:
 *   - Matrices are dense, row-major, float32, leading dimension = number of
 *     columns.  Row i of W is output coordinate i, column j input
 *     coordinate j.
 *   - Every pointer is a DEVICE pointer (hipMalloc'd or equivalent), owned by
 *     the caller.  The library never allocates device memory, never frees
 *     caller memory and never synchronises: all work is enqueued on `stream`
 *     in order and the call returns as soon as it is enqueued.
 *   - Scratch memory is the caller's `workspace` (device, >= 256-byte
 *     aligned, at least the size the matching *_workspace_bytes call
 *     returns).  Its contents are undefined after a call.  Two calls that
 *     share a workspace must be ordered (same stream or synchronised).
 *   - Return value: BAKRON_SUCCESS (0) when the work was enqueued, or a
 *     negative BAKRON_ERR_* code for an argument error detected on the
 *     host, in which case nothing was enqueued.  Numerical failures found on
 *     the device are reported through `info` (bakron_factor).
 *   - Inputs are const and are not modified.  Inputs and outputs must not
 *     overlap.
 */
#ifndef BAKRON_H
#define BAKRON_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BAKRON_SUCCESS 0
#define BAKRON_ERR_NULL_POINTER (-1) /* a required pointer is NULL */
#define BAKRON_ERR_BAD_SIZE (-2)     /* m or n negative or above BAKRON_MAX_DIM */
#define BAKRON_ERR_WORKSPACE (-3)    /* workspace NULL, too small or not 256-byte aligned */
#define BAKRON_ERR_BAD_ARG (-4)      /* damp_frac out of range, or a matrix pointer that
                                        must be 16-byte aligned is not */
#define BAKRON_ERR_HIP (-5)          /* a HIP launch call failed */
#define BAKRON_ERR_TOO_LARGE (-6)    /* the problem needs more scratch than the fixed
                                        maximum of bakron_solve_noalloc */

/* Largest supported m or n. */
#define BAKRON_MAX_DIM 65536

/* Version of this ABI (major * 10000 + minor * 100 + patch). */
int bakron_version(void);

/* Human-readable text for a return code (static storage, never NULL). */
const char* bakron_strerror(int code);

/*
 * Workspace bytes that bakron_factor needs for an n x n factor
 * (0 when n == 0).  Deterministic; does not touch the device.
 */
size_t bakron_factor_workspace_bytes(int64_t n);

/*
 * bakron_factor -- damping, reverse Cholesky and normalised inverse of one
 * Kronecker factor ([S] Corollary 3.4: L = RevCholesky(A)).
 *
 *   A_d = A + damp_frac * mean(diag A) * I           (damping; not on the pages,
 *                                                     GPTQ's usual 1% convention)
 *   L   lower triangular with A_d = L^T L           (RevCholesky)
 *   P   = L^-1 diag(L), unit lower triangular        (GPTQ's normalised inverse
 *                                                     rows for the factor)
 *
 * A      [in]  n x n, symmetric; only the lower triangle and the diagonal are
 *              read.  Not modified.
 * n      [in]  0 <= n <= BAKRON_MAX_DIM.  n == 0 enqueues nothing.
 * damp_frac [in] finite, >= 0 (use 0.01 for 1% damping).
 * L      [out] n x n; zeros above the diagonal.  16-byte aligned.
 * P      [out] n x n; ones on the diagonal, zeros above it.  16-byte aligned.
 * info   [out] one device int32: 0 on success, or k + 1 when the pivot of
 *              row k (0-based; rows are eliminated from the last upward) is
 *              not positive (A_d not positive definite or not finite), as in
 *              LAPACK.  Written on the device; read it after synchronising.
 *              L and P are undefined when info != 0.
 * workspace, workspace_bytes [in] scratch, >= bakron_factor_workspace_bytes(n).
 * stream [in]  HIP stream (0 = legacy default stream).  Factors of 8192 and
 *              more (whose top level runs on 128 x 128 blocks) also run part
 *              of the top level's products on one of the library-owned
 *              streams of bakron_solve, forked from and joined back into
 *              `stream` within the call: the result is ordered on `stream`
 *              like the rest.
 */
int bakron_factor(const float* A, int64_t n, float damp_frac, float* L, float* P,
                  int32_t* info, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * Workspace bytes that bakron_solve needs for an m x n weight
 * (0 when m == 0 or n == 0).  Deterministic; does not touch the device.
 */
size_t bakron_solve_workspace_bytes(int64_t m, int64_t n);

/*
 * bakron_solve -- the BaKron rounding of W under A (x) B ([S] derivation and
 * Theorem 3.2; [A] abstract).
 *
 * Computes the output of GPTQ run on vec(W) (column-major) with Hessian
 * A_d (x) B_d.  Equivalently: visit the entries in an order where (i, j)
 * comes after every (i', j') with i' <= i and j' <= j; at each entry take the
 * current working value w~, round it on the row's grid
 *     x = w~ / scale_i + zero_i,  c = clamp(rint(x), 0, maxq_i),
 *     v = scale_i (c - zero_i),   e = w~ - v,
 * and subtract e * P_B[i', i] * P_A[j', j] from every later entry
 * (i' >= i, j' >= j).  The solver groups entries into 64 x 64 tiles, sweeps
 * the tiles of one tile anti-diagonal in parallel (anti-diagonal
 * parallelism) and propagates the errors of the first half of the
 * remaining anti-diagonals to the second half with dense products
 * (recursive divide and conquer): O(m + n) dependent steps, O(mn(m + n))
 * work.  Arithmetic is float32; the rounding decision x is formed as
 * float32(w~ / scale) + zero.
 *
 * W        [in]  m x n.  Not modified.
 * m, n     [in]  0 <= m, n <= BAKRON_MAX_DIM; m == 0 or n == 0 enqueues
 *                nothing.  Any m, n (multiples of 64 avoid padding copies).
 * L_A, L_B [in]  n x n and m x m from bakron_factor(A), bakron_factor(B).
 *                Only their diagonals are read, and only when `objective`
 *                is not NULL (they may be NULL otherwise).
 * P_A, P_B [in]  n x n and m x m from bakron_factor; must be zero above the
 *                diagonal and one on it.  16-byte aligned.
 * scale    [in]  m floats, finite and > 0 (grid step of each output row).
 * zero     [in]  m floats, finite (zero point, fractional allowed).
 * maxq     [in]  m int32 in [1, 255] (largest code of each row).
 *                The grid contract is the caller's to keep: the grid is
 *                device memory and the library does not read it on the host
 *                (the Python binding's check_grid checks it before it
 *                enqueues anything).  Outside the contract the outputs are
 *                undefined (a maxq above 255 does not fit the uint8 codes).
 * V        [out] m x n float32, V_ij = scale_i (c_ij - zero_i).
 * codes    [out] m x n uint8 codes c_ij.
 * err      [out, nullable] m x n float32 raw errors e_ij = w~_ij - V_ij.
 * objective [out, nullable] one device double:
 *                sum_ij (L_B[i,i] L_A[j,j] e_ij)^2, which equals
 *                ||L_B (V - W) L_A^T||_F^2 ([S] Corollary 3.4's quantity).
 * workspace, workspace_bytes [in] scratch, >= bakron_solve_workspace_bytes(m, n).
 * stream   [in]  HIP stream of the current device.  All work is ordered on
 *                it: part of the propagation of the upper recursion levels
 *                runs on library-owned streams of the same device, forked
 *                from and joined back into `stream` with events before the
 *                call's last kernel, so later work on `stream` sees every
 *                result.  The library-owned streams are a fixed pool of four
 *                per device (created on first use, default priority, kept
 *                until the process ends); calls from different caller
 *                streams share them, so their side work runs in the order it
 *                was enqueued.  Two calls that share one workspace must be
 *                ordered on one stream.
 */
int bakron_solve(const float* W, int64_t m, int64_t n,
                 const float* L_A, const float* P_A,
                 const float* L_B, const float* P_B,
                 const float* scale, const float* zero, const int32_t* maxq,
                 float* V, uint8_t* codes, float* err, double* objective,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * bakron_solve_grouped -- bakron_solve with one grid per (output row, group of
 * group_size input columns) instead of one per row ([A] abstract: the base
 * quantizer is modular).  Entry (i, j) is rounded on grid entry
 * i * G + j / group_size of the arrays below, G = ceil(n / group_size)
 * (static groups: every grid is a fixed input, as the per-row grid is, so
 * the rounding rule of an entry does not depend on the order entries are
 * visited in and [S] Theorem 3.2 still holds; a caller typically computes
 * the grids from the original W's group slices).
 *
 * group_size [in] a positive multiple of 64 (BAKRON_ERR_BAD_ARG otherwise);
 *                 group_size >= n gives G = 1, the per-row case.
 * scale, zero, maxq [in] m x G row-major arrays, with the contract of
 *                 bakron_solve's per-row grid on every entry.
 * Everything else (arguments, workspace: bakron_solve_workspace_bytes,
 * streams, errors) is bakron_solve's.
 */
int bakron_solve_grouped(const float* W, int64_t m, int64_t n,
                         const float* L_A, const float* P_A,
                         const float* L_B, const float* P_B,
                         const float* scale, const float* zero, const int32_t* maxq,
                         int64_t group_size,
                         float* V, uint8_t* codes, float* err, double* objective,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes that bakron_solve_antidiagonal needs for an m x n weight
 * (0 when m == 0 or n == 0): two Mp x Np float buffers, an Np x Np one, a
 * padded Mp x Mp one when m is not a multiple of 64 and Mp doubles
 * (Mp, Np: m, n rounded up to 64).  Host only.
 */
size_t bakron_solve_antidiagonal_workspace_bytes(int64_t m, int64_t n);

/*
 * bakron_solve_antidiagonal -- BaKron-antidiagonal ([S] derivation, second
 * variant; Theorem 3.2; timed against BaKron in [S] Table 3): the same
 * rounding as bakron_solve, computed one entry anti-diagonal i + j = k at a
 * time.  The entries of D_k do not update one another, so they are rounded
 * together, and their raw errors E_k reach every later entry through one
 * rank-|D_k| product W~ -= P_B E_k P_A^T: m + n - 1 dependent steps but
 * about m^2 n^2 / 2 multiply-adds (bakron_solve's divide and conquer needs
 * mn(m + n) / 2).  The rounding rule and arithmetic of every entry are
 * bakron_solve's (float32, the decision float32(w~ / scale) + zero); the
 * products sum in another order, so codes may part from bakron_solve's only
 * where a decision lies within float32 rounding of a boundary.
 *
 * Arguments, grid contract and errors are those of bakron_solve; workspace:
 * bakron_solve_antidiagonal_workspace_bytes.  All work runs on `stream`
 * (two kernel launches per anti-diagonal).
 */
int bakron_solve_antidiagonal(const float* W, int64_t m, int64_t n,
                              const float* L_A, const float* P_A,
                              const float* L_B, const float* P_B,
                              const float* scale, const float* zero, const int32_t* maxq,
                              float* V, uint8_t* codes, float* err, double* objective,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Workspace bytes that bakron_quantize needs for an m x n weight (0 when
 * m or n is not positive or above BAKRON_MAX_DIM).  Host only.
 */
size_t bakron_quantize_workspace_bytes(int64_t m, int64_t n);

/*
 * bakron_quantize -- the whole BaKron rounding of one layer: bakron_factor(A),
 * bakron_factor(B) and bakron_solve in one call ([S] derivation, Theorem 3.2,
 * Corollary 3.4: the method takes W, the Kronecker factors A and B of the
 * Hessian and a grid, and returns the rounded weights).  The results equal
 * those of the three calls made one after the other.
 *
 * The two factorisations run on two of the library-owned streams of
 * bakron_solve (the fixed per-device pool), forked from `stream`.  When a dimension is a multiple of 64 and above 128,
 * its factorisation completes leading blocks [0, s)^2 of L and P one after
 * the other (s = the splits of its recursion on the leading half), and the
 * solve, on `stream`, runs each of its kernels as soon as the blocks that
 * hold its tiles are complete.  All outputs are complete for later work on
 * `stream`.
 *
 * W, m, n, scale, zero, maxq, V, codes, err, objective: as in bakron_solve.
 * A, B       [in]  n x n and m x m, as in bakron_factor.  Not modified.
 * damp_frac  [in]  as in bakron_factor, for both factors.
 * L_A, P_A, info_A [out] bakron_factor(A)'s outputs (n x n, 16-byte aligned).
 * L_B, P_B, info_B [out] bakron_factor(B)'s outputs (m x m, 16-byte aligned).
 * workspace, workspace_bytes [in] scratch, >= bakron_quantize_workspace_bytes.
 * stream     [in]  HIP stream of the current device.
 * Returns BAKRON_SUCCESS, or an error code for invalid arguments (nothing is
 * enqueued then) or a failed launch.
 */
int bakron_quantize(const float* W, int64_t m, int64_t n, const float* A, const float* B,
                    float damp_frac, const float* scale, const float* zero, const int32_t* maxq,
                    float* L_A, float* P_A, int32_t* info_A, float* L_B, float* P_B, int32_t* info_B,
                    float* V, uint8_t* codes, float* err, double* objective,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Batched solves of independent layers ([S]: every linear layer has its own
 * W, A and B, so layers share nothing).  One descriptor per layer; the
 * fields mean what the arguments of bakron_solve mean.
 */
typedef struct bakron_layer {
    const float* W;
    int64_t m, n;
    const float* L_A;
    const float* P_A;
    const float* L_B;
    const float* P_B;
    const float* scale;
    const float* zero;
    const int32_t* maxq;
    float* V;
    uint8_t* codes;
    float* err;          /* nullable */
    double* objective;   /* nullable */
} bakron_layer;

/*
 * Workspace bytes for bakron_solve_batch with these layers on n_streams
 * streams: one slice per stream, each as large as the largest workspace a
 * layer of that stream needs (layer k runs on stream k % n_streams), every
 * slice 256-byte aligned.  A batch layer runs entirely on its stream (no
 * library-owned streams), so its slice can be smaller than
 * bakron_solve_workspace_bytes.  0 when count or n_streams is not positive.
 * Host only.
 */
size_t bakron_solve_batch_workspace_bytes(const bakron_layer* layers, int32_t count, int32_t n_streams);

/*
 * bakron_solve_batch -- bakron_solve for `count` independent layers, spread
 * over the caller's streams: layer k is enqueued on streams[k % n_streams]
 * with that stream's workspace slice, so layers on one stream run in order
 * and layers on different streams may run concurrently.  Each layer's
 * results are those of bakron_solve on the same inputs (the same kernels,
 * all on the layer's stream).
 *
 * layers    [in]  host array of `count` descriptors (device pointers inside).
 * count     [in]  >= 0; 0 enqueues nothing.
 * workspace, workspace_bytes [in] scratch,
 *                 >= bakron_solve_batch_workspace_bytes(layers, count, n_streams).
 * streams   [in]  host array of n_streams HIP streams (1 <= n_streams <= 64).
 * Every descriptor is checked before anything is enqueued: a bad layer
 * returns the error bakron_solve would return for it, and nothing runs.
 */
int bakron_solve_batch(const bakron_layer* layers, int32_t count, void* workspace, size_t workspace_bytes,
                       const hipStream_t* streams, int32_t n_streams);

/*
 * Workspace bytes that bakron_gptq needs for an m x n weight
 * (0 when m == 0 or n == 0).  Deterministic; does not touch the device.
 */
size_t bakron_gptq_workspace_bytes(int64_t m, int64_t n);

/*
 * bakron_gptq -- the one-sided case B = I of bakron_solve, i.e. GPTQ with the
 * input-side Hessian A ([S] setup: GPTQ's Hessian is A (x) I; [N5]: GPTQ as
 * the one-sided comparison point).
 *
 * Returns what bakron_solve returns when P_B is the identity: with B = I an
 * error e at (i, j) only changes later columns of the same row i, by
 * -e P_A[j', j], so rows are independent and column j of every row is
 * rounded at step j (n dependent steps, O(m n^2) work).  The rounding rule,
 * the float32 arithmetic and the grid contract are those of bakron_solve.
 *
 * W        [in]  m x n.  Not modified.
 * m, n     [in]  0 <= m, n <= BAKRON_MAX_DIM; m == 0 or n == 0 enqueues
 *                nothing.  Any m, n.
 * L_A      [in]  n x n from bakron_factor(A); only its diagonal is read, and
 *                only when `objective` is not NULL (may be NULL otherwise).
 * P_A      [in]  n x n from bakron_factor(A); zero above the diagonal, one on
 *                it.  16-byte aligned.
 * scale, zero, maxq [in] as in bakron_solve (m entries each).
 * V, codes [out] m x n, as in bakron_solve.
 * err      [out, nullable] m x n raw errors.
 * objective [out, nullable] one device double: sum_ij (L_A[j,j] e_ij)^2,
 *                the objective of bakron_solve with L_B = I.
 * workspace, workspace_bytes [in] scratch, >= bakron_gptq_workspace_bytes(m, n).
 * stream   [in]  HIP stream.
 */
int bakron_gptq(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                const float* scale, const float* zero, const int32_t* maxq,
                float* V, uint8_t* codes, float* err, double* objective,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * bakron_gptq_grouped -- bakron_gptq with per-group grids, read as in
 * bakron_solve_grouped (group_size a positive multiple of 64; scale, zero and
 * maxq m x ceil(n / group_size) row-major).  Workspace:
 * bakron_gptq_workspace_bytes.
 */
int bakron_gptq_grouped(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                        const float* scale, const float* zero, const int32_t* maxq, int64_t group_size,
                        float* V, uint8_t* codes, float* err, double* objective,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Kronecker factors from per-sample inputs ([S], Hessian choices): with
 * input activations a_t (n) and output gradients b_t (m) of N samples,
 *   K-FAC-style independence:          A = E[a a^T],        B = E[b b^T];
 *   Shampoo-style, one power-iteration step of the nearest Kronecker
 *   product from the identity:         A = E[|b|^2 a a^T],  B = E[|a|^2 b b^T].
 * Both are weighted second moments of a sample-major matrix, built from the
 * two calls below (the weights |y_t|^2 come from bakron_row_sqnorms of the
 * other side's samples; scale = 1 / N).
 */

/*
 * bakron_row_sqnorms -- out[t] = sum_i X[t, i]^2 for t < N.
 *
 * X      [in]  N x n, row-major (row t = sample t); 16-byte aligned.
 * N, n   [in]  N >= 0, 0 <= n <= BAKRON_MAX_DIM, n a multiple of 4
 *              (BAKRON_ERR_BAD_ARG otherwise); N == 0 or n == 0 enqueues
 *              nothing.
 * out    [out] N floats.
 * stream [in]  HIP stream.
 */
int bakron_row_sqnorms(const float* X, int64_t N, int64_t n, float* out, hipStream_t stream);

/*
 * bakron_moment -- M = scale * sum_t w_t x_t x_t^T  (x_t = row t of X).
 *
 * X      [in]  N x n, row-major (row t = sample t); 16-byte aligned.
 * N, n   [in]  as in bakron_row_sqnorms; n == 0 enqueues nothing, N == 0
 *              writes zeros.
 * w      [in, nullable] N per-sample weights; NULL means w_t = 1 (K-FAC).
 * scale  [in]  finite (1 / N for an expectation).
 * M      [out] n x n.  The lower triangle and the diagonal are written, the
 *              strict upper triangle is not touched (bakron_factor reads
 *              only the lower triangle and the diagonal).
 * stream [in]  HIP stream.
 */
int bakron_moment(const float* X, int64_t N, int64_t n, const float* w, float scale, float* M,
                  hipStream_t stream);

/*
 * bakron_solve_noalloc -- bakron_solve with no workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It calls no hipMalloc,
 * hipFree or other allocating routine, creates no stream or event, and
 * enqueues only kernel launches on `stream`.
 *
 * Scratch: a file-scope device array of BAKRON_NOALLOC_SCRATCH_BYTES (256 MiB)
 * inside the library; each GPU the library runs on holds its own copy until
 * the process ends.  The problem fits when its unsplit solve workspace,
 * bakron_solve_batch_workspace_bytes of the one layer on one stream, is at
 * most that size (for m and n multiples of 64: 12 m n bytes plus a little,
 * e.g. up to 4096 x 4096); larger problems return BAKRON_ERR_TOO_LARGE and
 * enqueue nothing.  The scratch is looked up on the first call on each
 * device (with that device current).
 *
 * Every call on one GPU uses that GPU's one scratch array: calls that overlap
 * on one GPU (different streams not ordered against each other, or
 * different host threads) race and their results are undefined.  Calls
 * ordered on one stream are safe; nothing in the scratch must start at zero,
 * so a call does not depend on what the previous one left there.
 *
 * Arguments, results and errors are those of bakron_solve (the results are
 * bakron_solve's bit for bit), without workspace and workspace_bytes; all
 * work runs on `stream` itself (no library-owned streams).
 */
#define BAKRON_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

int bakron_solve_noalloc(const float* W, int64_t m, int64_t n,
                         const float* L_A, const float* P_A,
                         const float* L_B, const float* P_B,
                         const float* scale, const float* zero, const int32_t* maxq,
                         float* V, uint8_t* codes, float* err, double* objective,
                         hipStream_t stream);

/*
 * Profiling.  The *_profiled calls enqueue exactly the work of the plain
 * call, but launch every kernel with HIP start/stop events recorded around
 * it, then SYNCHRONISE `stream` and report, per kernel, the number of
 * launches, the summed kernel time and the summed algorithmic flops and
 * HBM bytes of those launches (the work the kernel's mathematical operation
 * needs: nonzero block products, each operand tile read once and each
 * output tile written once; padding and recomputation not counted).
 * For profilers and benchmarks; they create and destroy HIP events (host
 * objects) but allocate no device memory.
 *
 * stats     [out] host array of max_stats entries; filled in kernel order.
 * max_stats [in]  capacity (BAKRON_MAX_KERNEL_KINDS is always enough).
 * n_stats   [out] host int32: number of entries written (kernels launched).
 */
#define BAKRON_MAX_KERNEL_KINDS 48

typedef struct bakron_kernel_stat {
    const char* name;     /* kernel name (static storage) */
    int32_t launches;     /* launches of this kernel */
    double total_ms;      /* summed kernel time, milliseconds */
    double alg_flops;     /* summed algorithmic flops */
    double alg_bytes;     /* summed algorithmic HBM bytes */
} bakron_kernel_stat;

int bakron_factor_profiled(const float* A, int64_t n, float damp_frac, float* L, float* P,
                           int32_t* info, void* workspace, size_t workspace_bytes,
                           hipStream_t stream, bakron_kernel_stat* stats, int32_t max_stats,
                           int32_t* n_stats);

int bakron_solve_profiled(const float* W, int64_t m, int64_t n,
                          const float* L_A, const float* P_A,
                          const float* L_B, const float* P_B,
                          const float* scale, const float* zero, const int32_t* maxq,
                          float* V, uint8_t* codes, float* err, double* objective,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

int bakron_gptq_profiled(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                         const float* scale, const float* zero, const int32_t* maxq,
                         float* V, uint8_t* codes, float* err, double* objective,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

int bakron_solve_antidiagonal_profiled(const float* W, int64_t m, int64_t n,
                                       const float* L_A, const float* P_A,
                                       const float* L_B, const float* P_B,
                                       const float* scale, const float* zero, const int32_t* maxq,
                                       float* V, uint8_t* codes, float* err, double* objective,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                                       bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

int bakron_moment_profiled(const float* X, int64_t N, int64_t n, const float* w, float scale, float* M,
                           hipStream_t stream, bakron_kernel_stat* stats, int32_t max_stats,
                           int32_t* n_stats);

#ifdef __cplusplus
}
#endif

#endif /* BAKRON_H */
