// factor.hip -- damped reverse Cholesky and normalised inverse of one
// Kronecker factor, for gfx950.
//
// Computes L lower with A_d = L^T L ("RevCholesky" of the paper summary
// "FastKron: Efficient Quantization with Kronecker-Factored Hessians",
// Corollary 3.4) and P = L^-1 diag(L), where A_d = A + frac * mean(diag A) I.
//
// Algorithm: recursive blocked reverse Cholesky that carries the inverse
// along, so every O(n^3) step is a GEMM on the fp32 MFMA units.  With the
// index range split into a leading part 1 (n1) and a trailing part 2 (n2),
//   A = L^T L  gives  A22 = L22^T L22,  A21 = L22^T L21,
//                     A11 - L21^T L21 = L11^T L11,
// and the inverse of the block-lower L is
//   L^-1 = [[L11^-1, 0], [-L22^-1 L21 L11^-1, L22^-1]].
// So: recurse on 2 (gives L22 and Li22 = L22^-1); L21 = Li22^T A21 (GEMM,
// triangular left operand); A11 -= L21^T L21 (SYRK, lower blocks only);
// recurse on 1; Li21 = -Li22 (L21 Li11) (two GEMMs).  On the levels that use
// 64 x 64 tiles the last two products are grouped the other way,
// U = -Li22 L21 in the SYRK's launch and Li21 = U Li11 after the recursion
// on 1, so each node has one dependent launch fewer.  Diagonal blocks of 128
// (or 64) are factored and inverted in LDS by one workgroup.
//
// Buffers: Pbuf starts as A_d (lower part used) and ends as Li; Lbuf
// receives L.  Both are n x n with pitch ld.  The n2 x n1 temporary (T or U)
// lives in the workspace, one per depth of the recursion.  A final pass scales Li's columns by diag(L) (giving P)
// and writes zeros above both diagonals.  When n is a multiple of 64 (and
// above 128), the nodes of the leading spine (the blocks [0, nsz)^2) run that
// pass on their blocks as soon as these are final, and form their P21 from
// the finished P11 directly (see factor_rec), so a solve can start on the
// leading blocks while the rest of the factorisation runs.
#include <algorithm>
#include <memory>
#include <mutex>

#include "gemm.hpp"
#include "internal.hpp"

namespace bk {

// ---------------------------------------------------------------- damping

__global__ void k_clear_info(int32_t* __restrict__ info) { if (threadIdx.x == 0) info[0] = 0; }

__global__ __launch_bounds__(256) void k_diag_mean(const float* __restrict__ A, int64_t n,
                                                   float* __restrict__ mean_out)
{
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += (double)A[i * n + i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) mean_out[0] = (float)(red[0] / (double)n);
}

// dst (Np x Np, pitch ld) = lower triangle of A + frac * mean * I; identity on
// the padding diagonal, zeros elsewhere (the upper triangle is not read).
// Each thread writes four adjacent columns with one 16-byte store; rows of A
// are read with 16-byte loads where a group lies below the diagonal and A's
// rows are 16-byte aligned (vec), element by element elsewhere.
__global__ __launch_bounds__(256) void k_load_damped(const float* __restrict__ A, int64_t n,
                                                     float* __restrict__ dst, int64_t Np, int64_t ld,
                                                     const float* __restrict__ mean, float frac, int vec)
{
    // frac == 0 adds nothing (not 0 * mean, which is NaN for a non-finite diagonal)
    const float add = frac != 0.f ? frac * mean[0] : 0.f;
    for (int64_t i = blockIdx.y; i < Np; i += gridDim.y)
        for (int64_t j = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); j < Np; j += (int64_t)gridDim.x * 1024) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (vec && i < n && j + 3 < i && j + 3 < n) {
                v = *reinterpret_cast<const f32x4*>(A + i * n + j);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t c = j + q;
                    if (i < n && c < n) {
                        if (c < i) v[q] = A[i * n + c];
                        else if (c == i) v[q] = A[i * n + c] + add;
                    } else if (i == c) {
                        v[q] = 1.f;
                    }
                }
            }
            *reinterpret_cast<f32x4*>(dst + i * ld + j) = v;
        }
}

// --------------------------------------------------- diagonal blocks
//
// k_f_diag factors a whole diagonal block of 64 or 128 in one workgroup,
// with the block and its inverse resident in LDS (2 x 128 x 132 floats).
//
// Factor: right-looking over 16 x 16 diagonal blocks, last first.  For
// block b: one wave factors it (chol16: L_bb); then the panel
// L[b][0:16b] = L_bb^-T A[b][0:16b] is solved column by column (one thread
// per column, last row first), and the leading part is updated,
// A[0:16b][0:16b] -= L[b]^T L[b] (lower triangle).  This is A = L^T L
// eliminated from the last row up, 16 rows at a time.  The inverses of the
// 16-blocks are left out of this chain and formed afterwards.
//
// Inverse: the diagonal 16-blocks come from inv16; the off-diagonal part
// by the block rule L^-1 = [[X11, 0], [-X22 L21 X11, X22]] applied to 2 x 16,
// then 2 x 32, then 2 x 64 blocks (the last two on the MFMA units).  Each
// level parks T = L21 X11 in the upper block of its pair and clears it
// after use, since the next level multiplies whole (lower-triangular)
// blocks of X.

constexpr int kDP = 132;   // LDS pitch (floats) of the block and its inverse

// Threads of k_f_diag: wave 0 runs the pivot chain (chol16), the others the
// update of the upper-left part beside it and, after the factorisation, the
// 16 x 16 inverses (one round on eight waves, two on four).
#ifndef BAKRON_DIAG_THREADS
#define BAKRON_DIAG_THREADS 512
#endif
constexpr int kDiagThreads = BAKRON_DIAG_THREADS;
static_assert(kDiagThreads == 256 || kDiagThreads == 512, "four or eight waves");

// Issue priority of k_f_diag's waves over those of the products (the side
// stream's and the other factor's) where they share a CU.
#ifndef BAKRON_DIAG_PRIO
#define BAKRON_DIAG_PRIO 3
#endif
// ... and of the tile products launched on the chain (not the side stream's)
#ifndef BAKRON_CHAIN_PRIO
#define BAKRON_CHAIN_PRIO 2
#endif

// Value of v in lane `src` (any lane of the wave).
__device__ __forceinline__ float lane_get(float v, int src)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

__device__ __forceinline__ float wave_get(float v, int lane)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// chol16: reverse Cholesky S - U^T U = L^T L of the 16 x 16 block at S
// (pitch kDP, lower part read), by one wave with no LDS traffic between
// steps.  U (16 x 16, pitch kDP, may be null) is the block of the panel rows
// above S, whose update of S is applied here rather than by the leading-part
// update.  Lane 4i + q holds row i, columns 4q .. 4q + 3, of the symmetric
// working matrix (both triangles, so S[i][k] is in the lane's own quad).
// Step k (15 .. 0) takes row k from lanes 4k + q (ds_bpermute) and
// S[i][k] from the quad, and eliminates: S[i][j] -= S[i][k] S[k][j] /
// S[k][k] for i < k; rows stay unscaled and are scaled once at the end,
// L[i][j] = S[i][j] / sqrt(S[i][i]) (S[i][i] taken when row i was the pivot).
// Reciprocals and square roots use the hardware approximations (about one
// ulp): the factor is judged by its backward error, not by correct
// rounding.  L overwrites S (zeros above the diagonal).  Returns the block
// row of the first non-positive (or NaN) pivot met, or -1.
__device__ __forceinline__ int chol16(float* __restrict__ S, const float* __restrict__ U)
{
    const int lane = threadIdx.x & 63;
    const int i = lane >> 2, q = lane & 3, c0 = 4 * q;
    float s[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int j = c0 + u;
        s[u] = (j <= i) ? S[i * kDP + j] : S[j * kDP + i];
    }
    if (U) {
        float ui[16];
        f32x4 uj[16];
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
            ui[tt] = U[tt * kDP + i];
            uj[tt] = *reinterpret_cast<const f32x4*>(U + tt * kDP + c0);
        }
#pragma unroll
        for (int tt = 0; tt < 16; ++tt)
#pragma unroll
            for (int u = 0; u < 4; ++u) s[u] = fmaf(-ui[tt], uj[tt][u], s[u]);
    }
    int fail = -1;
    float mypiv = 1.f;
    // Two pivots (k, k - 1) per step: rows k and k - 1 arrive together, and
    // each lane applies pivot k to row k - 1 itself (rk1' = rk1 - (S[k][k-1] /
    // S[k][k]) rk) before eliminating both, which halves the dependent chain.
    // Column k lives in register k % 4 of the quad's lane k / 4.
    auto chol2 = [&](const int k, const int ru, const int ru1) {   // ru = k % 4, ru1 = (k - 1) % 4
        float rk[4], rk1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            rk[u] = lane_get(s[u], 4 * k + q);
            rk1[u] = lane_get(s[u], 4 * (k - 1) + q);
        }
        const int g = k >> 2;                                        // k and k - 1 share the quad lane
        const float a = wave_get(s[ru], 4 * k + g);                  // S[k][k]
        const float bk = wave_get(s[ru1], 4 * k + g);                // S[k][k-1]
        const float c = wave_get(s[ru1], 4 * (k - 1) + g);           // S[k-1][k-1]
        const float sik = lane_get(s[ru], (lane & ~3) + g);          // S[i][k]
        const float sik1 = lane_get(s[ru1], (lane & ~3) + g);        // S[i][k-1]
        const float ia = __builtin_amdgcn_rcpf(a);
        const float cp = c - bk * bk * ia;                           // pivot k - 1 after pivot k
        if (!(a > 0.f) && fail < 0) fail = k;
        if (!(cp > 0.f) && fail < 0) fail = k - 1;
        if (i == k) mypiv = a;
        if (i == k - 1) mypiv = cp;
        const float m1 = (i < k) ? sik * ia : 0.f;
        const float m2 = (i < k - 1) ? (sik1 - sik * bk * ia) * __builtin_amdgcn_rcpf(cp) : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float r1p = fmaf(-bk * ia, rk[u], rk1[u]);
            s[u] = fmaf(-m2, r1p, fmaf(-m1, rk[u], s[u]));
        }
    };
#pragma unroll
    for (int g = 3; g >= 0; --g) {   // unrolled: lane indices and exchange addresses are constants
        chol2(4 * g + 3, 3, 2);
        chol2(4 * g + 1, 1, 0);
    }
    const float rs = __builtin_amdgcn_rsqf(mypiv);   // 1 / L[i][i]
#pragma unroll
    for (int u = 0; u < 4; ++u) S[i * kDP + c0 + u] = (c0 + u <= i) ? s[u] * rs : 0.f;
    return fail;
}

// inv16: X = L^-1 for the 16 x 16 lower-triangular L at S (pitch kDP), by one
// wave, in chol16's lane layout.  It solves L X = I by rows, forward: with
// R[i] = L[i][i] X[i], R[i] = e_i - sum_{k<i} (L[i][k] / L[k][k]) R[k], one
// row broadcast a step.  X gets zeros above its diagonal.
__device__ __forceinline__ void inv16(const float* __restrict__ S, float* __restrict__ X)
{
    const int lane = threadIdx.x & 63;
    const int i = lane >> 2, q = lane & 3, c0 = 4 * q;
    float l[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) l[u] = S[i * kDP + c0 + u];
    const float rs = __builtin_amdgcn_rcpf(S[i * kDP + i]);   // 1 / L[i][i]
    float r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = (c0 + u == i) ? 1.f : 0.f;
    // Two rows (k, k + 1) per step: R[k + 1] takes R[k]'s contribution
    // locally first.
    auto inv2 = [&](const int k, const int ru, const int ru1) {    // ru = k % 4, ru1 = (k + 1) % 4
        float rk[4], rk1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            rk[u] = lane_get(r[u], 4 * k + q);
            rk1[u] = lane_get(r[u], 4 * (k + 1) + q);
        }
        const int g = k >> 2;
        const float lkk = wave_get(l[ru], 4 * k + g);                // L[k][k]
        const float lk1k = wave_get(l[ru], 4 * (k + 1) + g);         // L[k+1][k]
        const float lk1k1 = wave_get(l[ru1], 4 * (k + 1) + g);       // L[k+1][k+1]
        const float lik = lane_get(l[ru], (lane & ~3) + g);          // L[i][k]
        const float lik1 = lane_get(l[ru1], (lane & ~3) + g);        // L[i][k+1]
        const float ik = __builtin_amdgcn_rcpf(lkk);
        const float c1 = (i > k) ? lik * ik : 0.f;
        const float c2 = (i > k + 1) ? lik1 * __builtin_amdgcn_rcpf(lk1k1) : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float r1p = fmaf(-lk1k * ik, rk[u], rk1[u]);
            r[u] = fmaf(-c2, r1p, fmaf(-c1, rk[u], r[u]));
        }
    };
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        inv2(4 * g, 0, 1);
        inv2(4 * g + 2, 2, 3);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) X[i * kDP + c0 + u] = (c0 + u <= i) ? r[u] * rs : 0.f;
}

// MFMA fragment of LDS operand element (r, k .. k + 3) (pitch kDP):
// RowK p[r * kDP + k], KRow p[k * kDP + r].
template <int LAYOUT>
__device__ __forceinline__ f32x4 ldsfrag(const float* p, int r, int k)
{
    if (LAYOUT == RowK) return *reinterpret_cast<const f32x4*>(p + r * kDP + k);
    return f32x4{p[k * kDP + r], p[(k + 1) * kDP + r], p[(k + 2) * kDP + r], p[(k + 3) * kDP + r]};
}

// One wave: the 32 x 32 tile of A B over K (a multiple of 8), A(r, k) and
// B(k, c) addressed as ldsfrag's (r, k) and (c, k).
template <int ALAY, int BLAY>
__device__ __forceinline__ f32x16 lds_mm32(const float* A, const float* B, int K)
{
    const int lane = threadIdx.x & 63;
    const int ml = lane & 31, k4 = 4 * (lane >> 5);
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    for (int kc = 0; kc < K; kc += 8) {
        const f32x4 a = ldsfrag<ALAY>(A, ml, kc + k4);
        const f32x4 b = ldsfrag<BLAY>(B, ml, kc + k4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
    }
    return acc;
}

// C (32 x 32 in LDS) = alpha * acc, one wave.
__device__ __forceinline__ void lds_put32(float* C, const f32x16& acc, float alpha)
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) C[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kDP + col] = alpha * acc[r];
}

// 64 x 64 x 64 product from LDS: wave w returns the 32 x 32 quadrant at rows
// 32 (w >> 1), columns 32 (w & 1) of A B.
template <int ALAY, int BLAY>
__device__ __forceinline__ f32x16 lds_mm64(const float* A, const float* B)
{
    const int wave = threadIdx.x >> 6;
    const int ro = 32 * (wave >> 1), co = 32 * (wave & 1);
    const float* Aw = (ALAY == RowK) ? A + ro * kDP : A + ro;
    const float* Bw = (BLAY == RowK) ? B + co * kDP : B + co;
    return lds_mm32<ALAY, BLAY>(Aw, Bw, 64);
}

__device__ __forceinline__ void lds_put64(float* C, const f32x16& acc, float alpha)
{
    const int wave = threadIdx.x >> 6;
    lds_put32(C + 32 * (wave >> 1) * kDP + 32 * (wave & 1), acc, alpha);
}

// One wave: X21 = -X22 (L21 X11) for 16 x 16 blocks at diagonal offset d
// (block rows d .. d + 31 of the 32-block); T goes to X's upper block.
__device__ __forceinline__ void inv_merge16(const float* sA, float* sX, int d)
{
    const int lane = threadIdx.x & 63;
    const int r = lane >> 2, c0 = 4 * (lane & 3);
    const float* L21 = sA + (d + 16) * kDP + d;
    const float* X11 = sX + d * kDP + d;
    const float* X22 = sX + (d + 16) * kDP + d + 16;
    float* T = sX + d * kDP + d + 16;          // upper block, unused by the result
    float* X21 = sX + (d + 16) * kDP + d;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float a = L21[r * kDP + k];
        const f32x4 b = *reinterpret_cast<const f32x4*>(X11 + k * kDP + c0);
        acc[0] = fmaf(a, b.x, acc[0]);
        acc[1] = fmaf(a, b.y, acc[1]);
        acc[2] = fmaf(a, b.z, acc[2]);
        acc[3] = fmaf(a, b.w, acc[3]);
    }
    *reinterpret_cast<f32x4*>(T + r * kDP + c0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const float a = X22[r * kDP + k];
        const f32x4 b = *reinterpret_cast<const f32x4*>(T + k * kDP + c0);
        acc[0] = fmaf(a, b.x, acc[0]);
        acc[1] = fmaf(a, b.y, acc[1]);
        acc[2] = fmaf(a, b.z, acc[2]);
        acc[3] = fmaf(a, b.w, acc[3]);
    }
    *reinterpret_cast<f32x4*>(X21 + r * kDP + c0) = f32x4{-acc[0], -acc[1], -acc[2], -acc[3]};
    // the next level multiplies whole blocks of X: its upper part must be zero
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    *reinterpret_cast<f32x4*>(T + r * kDP + c0) = f32x4{0.f, 0.f, 0.f, 0.f};
}

// A[r0 .. r0+3][cc .. cc+3] -= sum over the 16 panel rows t of Pr[t][r] Pr[t][c].
__device__ __forceinline__ void syrk_tile4(float* __restrict__ sA, const float* __restrict__ Pr, int r0, int cc)
{
    float acc[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(Pr + tt * kDP + r0);
        const f32x4 c = *reinterpret_cast<const f32x4*>(Pr + tt * kDP + cc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            acc[0][v] = fmaf(a.x, c[v], acc[0][v]);
            acc[1][v] = fmaf(a.y, c[v], acc[1][v]);
            acc[2][v] = fmaf(a.z, c[v], acc[2][v]);
            acc[3][v] = fmaf(a.w, c[v], acc[3][v]);
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4* p = reinterpret_cast<f32x4*>(sA + (r0 + u) * kDP + cc);
        f32x4 v = *p;
        v.x -= acc[u][0];
        v.y -= acc[u][1];
        v.z -= acc[u][2];
        v.w -= acc[u][3];
        *p = v;
    }
}

__global__ __launch_bounds__(kDiagThreads) void k_f_diag(float* __restrict__ Lbuf, float* __restrict__ Pbuf, int64_t ld,
                                                int64_t o, int nb, int32_t* __restrict__ info)
{
    if (BAKRON_DIAG_PRIO > 0) __builtin_amdgcn_s_setprio(BAKRON_DIAG_PRIO);   // the chain's latency-bound step
    __shared__ __align__(16) float sA[128 * kDP];   // the block, then L
    __shared__ __align__(16) float sX[128 * kDP];   // L^-1
    __shared__ int sfail;
    const int t = threadIdx.x, wave = t >> 6;
    const int nf4 = nb / 4;
    {   // all global loads in flight before the LDS stores
        constexpr int NU = 128 * 128 / 4 / kDiagThreads;
        f32x4 v[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int f = t + kDiagThreads * u;
            if (f < nb * nf4) v[u] = *reinterpret_cast<const f32x4*>(Pbuf + (o + f / nf4) * ld + o + 4 * (f % nf4));
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int f = t + kDiagThreads * u;
            if (f < nb * nf4) *reinterpret_cast<f32x4*>(sA + (f / nf4) * kDP + 4 * (f % nf4)) = v[u];
        }
    }
    if (t == 0) sfail = -1;
    __syncthreads();

    // factor, 16 rows at a time from the bottom, with a one-block lookahead:
    // once the panel of block b is formed, wave 0 factors diagonal block
    // b - 1 (chol16, which applies that block's share of the update itself)
    // while waves 1 - 7 apply the rest of block b's update to the remaining
    // upper-left part.
    if (wave == 0) {
        const int b = nb / 16 - 1;
        const int f = chol16(sA + 16 * b * (kDP + 1), nullptr);
        if (t == 0 && f >= 0) sfail = 16 * b + f;
    }
    __syncthreads();
    for (int b = nb / 16 - 1; b >= 1; --b) {
        const int W = 16 * b;
        float* Pr = sA + W * kDP;                    // rows of block b
        if (t < W) {   // panel: solve L_bb^T Z = Pr for column t, from the last row up
            const float* Lbb = sA + W * (kDP + 1);
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = Pr[r * kDP + t];
            // L_bb's lower triangle (the same for every lane) and the
            // reciprocals of its diagonal, all read before the substitution,
            // whose dependent chain is then one multiply and one fma a row
            f32x4 lr[16][4];
            float rd[16];
#pragma unroll
            for (int tt = 15; tt >= 0; --tt)
#pragma unroll
                for (int v = 0; v <= tt / 4; ++v) lr[tt][v] = *reinterpret_cast<const f32x4*>(Lbb + tt * kDP + 4 * v);
#pragma unroll
            for (int tt = 15; tt >= 0; --tt) rd[tt] = __builtin_amdgcn_rcpf(lr[tt][tt / 4][tt % 4]);
#pragma unroll
            for (int tt = 15; tt >= 0; --tt) {
                p[tt] *= rd[tt];
#pragma unroll
                for (int r = 0; r < tt; ++r) p[r] = fmaf(-lr[tt][r / 4][r % 4], p[tt], p[r]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) Pr[r * kDP + t] = p[r];
        }
        __syncthreads();
        // A[0:W][0:W] -= Pr^T Pr on the 4 x 4 tiles of the lower triangle;
        // the tiles of diagonal block b - 1 (rows and columns W - 16 .. W - 1)
        // are left to wave 0's chol16
        const int n4 = W / 4, ntile = n4 * (n4 + 1) / 2;
        const int d4 = n4 - 4;                       // first 4-row of block b - 1
        if (wave == 0) {
            const int f = chol16(sA + 16 * (b - 1) * (kDP + 1), Pr + W - 16);
            if (t == 0 && f >= 0 && sfail < 0) sfail = 16 * (b - 1) + f;
        } else {
            for (int idx = t - 64; idx < ntile; idx += kDiagThreads - 64) {
                int br = (int)((sqrtf(8.f * idx + 1.f) - 1.f) * 0.5f);
                while ((br + 1) * (br + 2) / 2 <= idx) ++br;
                while (br * (br + 1) / 2 > idx) --br;
                const int bc = idx - br * (br + 1) / 2;
                if (br >= d4 && bc >= d4) continue;  // wave 0's
                syrk_tile4(sA, Pr, 4 * br, 4 * bc);
            }
        }
        __syncthreads();
    }

    // inverse: the 16-blocks (inv16, one wave each), then merged pairs of
    // 2 x 16 blocks (one wave each), 2 x 32 (MFMA, one wave each), 2 x 64
    // (MFMA, four waves); T goes to the upper block of each pair
    for (int k = wave; k < nb / 16; k += kDiagThreads / 64) inv16(sA + 16 * k * (kDP + 1), sX + 16 * k * (kDP + 1));
    __syncthreads();
    if (wave < nb / 32) inv_merge16(sA, sX, 32 * wave);
    __syncthreads();
    if (wave < nb / 64) {
        const int d = 64 * wave;
        const f32x16 acc = lds_mm32<RowK, KRow>(sA + (d + 32) * kDP + d, sX + d * kDP + d, 32);   // L21 X11
        lds_put32(sX + d * kDP + d + 32, acc, 1.f);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const f32x16 acc2 = lds_mm32<RowK, KRow>(sX + (d + 32) * (kDP + 1), sX + d * kDP + d + 32, 32);
        lds_put32(sX + (d + 32) * kDP + d, acc2, -1.f);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x16 z;
#pragma unroll
        for (int q = 0; q < 16; ++q) z[q] = 0.f;
        lds_put32(sX + d * kDP + d + 32, z, 1.f);   // clear T: X's upper part must be zero for the next level
    }
    __syncthreads();
    if (nb == 128) {   // on the first four waves
        if (wave < 4) {
            const f32x16 acc = lds_mm64<RowK, KRow>(sA + 64 * kDP, sX);                  // T = L21 X11
            lds_put64(sX + 64, acc, 1.f);
        }
        __syncthreads();
        if (wave < 4) {
            const f32x16 acc2 = lds_mm64<RowK, KRow>(sX + 64 * (kDP + 1), sX + 64);       // X21 = -X22 T
            lds_put64(sX + 64 * kDP, acc2, -1.f);
        }
        __syncthreads();
    }

    for (int f = t; f < nb * nf4; f += kDiagThreads) {
        const int r = f / nf4, c = 4 * (f % nf4);
        f32x4 l = *reinterpret_cast<const f32x4*>(sA + r * kDP + c);
        f32x4 x = *reinterpret_cast<const f32x4*>(sX + r * kDP + c);
        if (c + 0 > r) l.x = x.x = 0.f;
        if (c + 1 > r) l.y = x.y = 0.f;
        if (c + 2 > r) l.z = x.z = 0.f;
        if (c + 3 > r) l.w = x.w = 0.f;
        *reinterpret_cast<f32x4*>(Lbuf + (o + r) * ld + o + c) = l;
        *reinterpret_cast<f32x4*>(Pbuf + (o + r) * ld + o + c) = x;
    }
    if (t == 0 && sfail >= 0) atomicCAS(info, 0, (int32_t)(o + sfail + 1));
}

// ------------------------------------------------------ recursive GEMMs

constexpr int FBM = 128, FBN = 128;   // 128 x 128 output blocks
// A level with fewer 128 x 128 blocks than this uses 64 x 64 tiles (k_f_tile).
#ifndef BAKRON_FACTOR_BLOCK_MIN
#define BAKRON_FACTOR_BLOCK_MIN 1024
#endif
constexpr int64_t kFactorBlockMin = BAKRON_FACTOR_BLOCK_MIN;

// L21 = Li22^T A21 : (n2 x n1); Li22^T is upper triangular, so output rows
// from r0 need K in [r0, n2).
__global__ __launch_bounds__(256) void k_f_panel(const float* __restrict__ Pbuf, float* __restrict__ Lbuf,
                                                 int64_t ld, int64_t o1, int64_t o2, int n1, int n2)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, KRow, KRow>::LDS_FLOATS];
    const int r0 = blockIdx.y * FBM, c0 = blockIdx.x * FBN;
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, KRow, KRow>(Pbuf + o2 * ld + o2 + r0, ld, n2 - r0,
                                 Pbuf + o2 * ld + o1 + c0, ld, n1 - c0, r0, n2, lds, acc);
    block_store<2, 2>(Lbuf + (o2 + r0) * ld + o1 + c0, ld, n2 - r0, n1 - c0, 1.f, 0.f, acc);
}

// T = L21 Li11 : (n2 x n1); Li11 is lower, so output columns from c0 need
// K in [c0, n1).  Row blocks run along x (the fast launch dimension), so
// the longest column blocks start first.
__global__ __launch_bounds__(256) void k_f_right(const float* __restrict__ Lbuf, const float* __restrict__ Pbuf,
                                                 float* __restrict__ T, int64_t ld, int64_t o1, int64_t o2,
                                                 int n1, int n2)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, RowK, KRow>::LDS_FLOATS];
    const int r0 = blockIdx.x * FBM, c0 = blockIdx.y * FBN;
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, RowK, KRow>(Lbuf + (o2 + r0) * ld + o1, ld, n2 - r0,
                                 Pbuf + o1 * ld + o1 + c0, ld, n1 - c0, c0, n1, lds, acc);
    block_store<2, 2>(T + (int64_t)r0 * n1 + c0, n1, n2 - r0, n1 - c0, 1.f, 0.f, acc);
}

// Li21 = -Li22 T : (n2 x n1); Li22 is lower, so output rows up to r0 + 127
// need K in [0, min(r0 + 128, n2)).
__global__ __launch_bounds__(256) void k_f_left(const float* __restrict__ T, float* __restrict__ Pbuf,
                                                int64_t ld, int64_t o1, int64_t o2, int n1, int n2)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, RowK, KRow>::LDS_FLOATS];
    // heaviest (largest K, last row blocks) first
    const int r0 = (int)(gridDim.y - 1 - blockIdx.y) * FBM, c0 = blockIdx.x * FBN;
    const int kend = min(r0 + FBM, n2);
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, RowK, KRow>(Pbuf + (o2 + r0) * ld + o2, ld, n2 - r0,
                                 T + c0, n1, n1 - c0, 0, kend, lds, acc);
    block_store<2, 2>(Pbuf + (o2 + r0) * ld + o1 + c0, ld, n2 - r0, n1 - c0, -1.f, 0.f, acc);
}

// A[ro + r][co + c] -= sum_{k < nk} L[ko + k][ro + r] L[ko + k][co + c] over
// the nr x nc rectangle (the update of pending columns co .. co + nc - 1 by
// the finished rows ko .. ko + nk - 1; see factor_rec).
__global__ __launch_bounds__(256) void k_f_update(const float* __restrict__ Lbuf, float* __restrict__ Pbuf,
                                                  int64_t ld, int64_t ro, int64_t co, int64_t ko, int nr, int nc,
                                                  int nk)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, KRow, KRow>::LDS_FLOATS];
    const int r0 = blockIdx.y * FBM, c0 = blockIdx.x * FBN;
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, KRow, KRow>(Lbuf + ko * ld + ro + r0, ld, nr - r0, Lbuf + ko * ld + co + c0, ld, nc - c0, 0, nk,
                                 lds, acc);
    block_store<2, 2>(Pbuf + (ro + r0) * ld + co + c0, ld, nr - r0, nc - c0, -1.f, 1.f, acc);
}

// The top level's T and Li21 products while a solve runs beside them on the
// factor's leading block (factor_enqueue with `lead`): at most kLeadGrid
// workgroups, each looping over blocks q = blockIdx.x, + gridDim.x, ... in
// the order of the plain launch (q = x + nx y), and each reserving enough LDS
// (dynamic, kLeadPad bytes) that no leaf of the solve fits beside it.  Two
// factors at once then leave 256 - 2 kLeadGrid CUs to the solve's leaves.
#ifndef BAKRON_LEAD_GRID
#define BAKRON_LEAD_GRID 96
#endif
constexpr unsigned kLeadGrid = BAKRON_LEAD_GRID;
// That grid suits top nodes whose products finish beside the solve's first
// subtree on it: at 8192 (1024 blocks) they take about 3.5 ms there against
// about 3.9 ms of solve.  A larger top node (14336: 3136 blocks) would take
// about five times longer than the subtree on 96 workgroups, so its products
// get kLeadGridBig workgroups instead, one per CU on most of the GPU, and
// leave the rest of the CUs to the solve's first leaves (at 4096 x 14336 the
// fused call then takes 52.7-53.1 ms, against 54.5 ms with the products on
// the full grid and 62 ms on 96 workgroups; 208-224 workgroups were best,
// 160 or 240 and more no better than the full grid).
#ifndef BAKRON_LEAD_MAX_BLOCKS
#define BAKRON_LEAD_MAX_BLOCKS 1024
#endif
constexpr unsigned kLeadMaxBlocks = BAKRON_LEAD_MAX_BLOCKS;
#ifndef BAKRON_LEAD_GRID_BIG
#define BAKRON_LEAD_GRID_BIG 224
#endif
constexpr unsigned kLeadGridBig = BAKRON_LEAD_GRID_BIG;   // 0: the full grid for larger top nodes
constexpr size_t kLeadPad = 160 * 1024 - kLeafLdsBytes - sizeof(float) * Gemm<2, 2, RowK, KRow>::LDS_FLOATS + 1024;

__global__ __launch_bounds__(256) void k_f_right_lead(const float* __restrict__ Lbuf, const float* __restrict__ Pbuf,
                                                      float* __restrict__ T, int64_t ld, int64_t o1, int64_t o2,
                                                      int n1, int n2, unsigned nx, unsigned count)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, RowK, KRow>::LDS_FLOATS];
    extern __shared__ float reserve[];
    (void)reserve;
    for (unsigned q = blockIdx.x; q < count; q += gridDim.x) {
        const int r0 = (int)(q % nx) * FBM, c0 = (int)(q / nx) * FBN;
        Acc acc;
        acc_zero(acc);
        block_gemm<2, 2, RowK, KRow>(Lbuf + (o2 + r0) * ld + o1, ld, n2 - r0,
                                     Pbuf + o1 * ld + o1 + c0, ld, n1 - c0, c0, n1, lds, acc);
        block_store<2, 2>(T + (int64_t)r0 * n1 + c0, n1, n2 - r0, n1 - c0, 1.f, 0.f, acc);
    }
}

__global__ __launch_bounds__(256) void k_f_left_lead(const float* __restrict__ T, float* __restrict__ Pbuf,
                                                     int64_t ld, int64_t o1, int64_t o2, int n1, int n2,
                                                     unsigned nx, unsigned ny, unsigned count)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, RowK, KRow>::LDS_FLOATS];
    extern __shared__ float reserve[];
    (void)reserve;
    for (unsigned q = blockIdx.x; q < count; q += gridDim.x) {
        const int r0 = (int)(ny - 1 - q / nx) * FBM, c0 = (int)(q % nx) * FBN;
        const int kend = min(r0 + FBM, n2);
        Acc acc;
        acc_zero(acc);
        block_gemm<2, 2, RowK, KRow>(Pbuf + (o2 + r0) * ld + o2, ld, n2 - r0,
                                     T + c0, n1, n1 - c0, 0, kend, lds, acc);
        block_store<2, 2>(Pbuf + (o2 + r0) * ld + o1 + c0, ld, n2 - r0, n1 - c0, -1.f, 0.f, acc);
    }
}

// The products with one 64 x 64 output tile per workgroup (one 32 x 32
// quadrant per wave) for the levels whose 128 x 128 grids are too small to
// fill the GPU.  There the inverse block is grouped as
// Li21 = (-Li22 L21) Li11: U = -Li22 L21 needs only the panel, so it shares
// one launch with the SYRK, and one product U Li11 is left for after the
// leading block's factorisation.  MODE: 0 panel; 1 syrk; 2 Li21 = U Li11;
// 3 syrk (first tb (tb + 1) / 2 workgroups) and U = -Li22 L21; 4 U alone
// (a right-looking node, whose SYRK ran in pieces).  T is U (n2 x n1,
// leading dimension n1).
template <int MODE>
__global__ __launch_bounds__(256) void k_f_tile(float* __restrict__ Lbuf, float* __restrict__ Pbuf,
                                                float* __restrict__ T, int64_t ld, int64_t o1, int64_t o2,
                                                int n1, int n2, int chain)
{
    if (BAKRON_CHAIN_PRIO > 0 && chain) __builtin_amdgcn_s_setprio(BAKRON_CHAIN_PRIO);   // on the factor's chain
    __shared__ __align__(16) float lds[kLds64];
    int r0, c0;
    bool syrk = (MODE == 1);
    if (MODE == 3 || MODE == 4) {
        const int tb = n1 / 64;
        const int q = (int)blockIdx.x - (MODE == 3 ? tb * (tb + 1) / 2 : 0);
        syrk = q < 0;
        if (!syrk) {   // U tiles, heaviest (largest K, last row tiles) first
            r0 = 64 * (n2 / 64 - 1 - q / tb);
            c0 = 64 * (q % tb);
        }
    }
    if (syrk) {   // linear index -> lower-triangular tile (br >= bc)
        const int q = blockIdx.x;
        int br = (int)((sqrtf(8.f * q + 1.f) - 1.f) * 0.5f);
        while ((br + 1) * (br + 2) / 2 <= q) ++br;
        while (br * (br + 1) / 2 > q) --br;
        r0 = 64 * br;
        c0 = 64 * (q - br * (br + 1) / 2);
    } else if (MODE == 2) {   // rows along x: the longest column tiles first
        r0 = 64 * (int)blockIdx.x;
        c0 = 64 * (int)blockIdx.y;
    } else if (MODE == 0) {
        r0 = 64 * (int)blockIdx.y;
        c0 = 64 * (int)blockIdx.x;
    }
    const int wave = threadIdx.x >> 6;
    const int qr = 32 * (wave >> 1), qc = 32 * (wave & 1);
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    if (MODE == 0) {          // L21 = Li22^T A21, K in [r0, n2)
        block_gemm64<KRow, KRow>(Pbuf + o2 * ld + o2 + r0, ld, Pbuf + o2 * ld + o1 + c0, ld, r0, n2, lds, acc);
        wave_store32(Lbuf + (o2 + r0 + qr) * ld + o1 + c0 + qc, ld, 1.f, 0.f, acc);
    } else if (MODE == 2) {   // Li21 = U Li11, K in [c0, n1)
        block_gemm64<RowK, KRow>(T + (int64_t)r0 * n1, n1, Pbuf + o1 * ld + o1 + c0, ld, c0, n1, lds, acc);
        wave_store32(Pbuf + (o2 + r0 + qr) * ld + o1 + c0 + qc, ld, 1.f, 0.f, acc);
    } else if (syrk) {        // A11 -= L21^T L21, lower part
        block_gemm64<KRow, KRow>(Lbuf + o2 * ld + o1 + r0, ld, Lbuf + o2 * ld + o1 + c0, ld, 0, n2, lds, acc);
        wave_store32(Pbuf + (o1 + r0 + qr) * ld + o1 + c0 + qc, ld, -1.f, 1.f, acc, (c0 + qc) - (r0 + qr));
    } else {                  // U = -Li22 L21, K in [0, r0 + 64)
        block_gemm64<RowK, KRow>(Pbuf + (o2 + r0) * ld + o2, ld, Lbuf + o2 * ld + o1 + c0, ld, 0, r0 + 64, lds, acc);
        wave_store32(T + (int64_t)(r0 + qr) * n1 + c0 + qc, n1, -1.f, 0.f, acc);
    }
}

// P = Li diag(L) on and below the diagonal, zeros above, for L and P; when
// the factor ran in padded workspace, also copy the leading n x n out.
// Each thread owns four adjacent columns for a stripe of rows, so the
// diagonal entries it scales by are read once.
__global__ __launch_bounds__(256) void k_f_finish(float* __restrict__ Lbuf, float* __restrict__ Pbuf, int64_t ld,
                                                  int64_t i0, int64_t i1, int64_t j0, int64_t j1, int64_t n,
                                                  float* __restrict__ Lout, float* __restrict__ Pout)
{
    const int64_t j = j0 + 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (j >= j1) return;
    float dg[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) dg[q] = Lbuf[(j + q) * ld + j + q];
    for (int64_t i = i0 + blockIdx.y; i < i1; i += gridDim.y) {
        f32x4 l = {0.f, 0.f, 0.f, 0.f}, p = {0.f, 0.f, 0.f, 0.f};
        if (j <= i) {
            l = *reinterpret_cast<const f32x4*>(Lbuf + i * ld + j);
            p = *reinterpret_cast<const f32x4*>(Pbuf + i * ld + j);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool below = j + q <= i;
                l[q] = below ? l[q] : 0.f;
                p[q] = below ? p[q] * dg[q] : 0.f;
            }
        }
        if (Lout) {
            if (i < n)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (j + q < n) {
                        Lout[i * n + j + q] = l[q];
                        Pout[i * n + j + q] = p[q];
                    }
        } else {
            *reinterpret_cast<f32x4*>(Lbuf + i * ld + j) = l;
            *reinterpret_cast<f32x4*>(Pbuf + i * ld + j) = p;
        }
    }
}

// ------------------------------------------------------------ host side

namespace {

// Depths of the recursion: sizes halve from at most kMaxDim down to 2 kTile.
constexpr int kFactorDepths = 16;

struct FactorPlan {
    int64_t n, Np;
    bool padded;
    size_t off_mean, off_T, off_L, off_P, total;
    int64_t tbase[kFactorDepths];   // offset (floats) of each depth's n2 x n1 product buffer within T
};

// Largest n1 n2 of the nodes at each depth (the split of factor_rec).
void depth_products(int64_t nsz, int d, int64_t* most)
{
    if (nsz <= 2 * kTile) return;
    const int64_t nt = nsz / kTile, n1 = kTile * (nt / 2), n2 = nsz - n1;
    most[d] = std::max(most[d], n1 * n2);
    depth_products(n2, d + 1, most);
    if (n1 != n2) depth_products(n1, d + 1, most);
}

FactorPlan plan_factor(int64_t n)
{
    FactorPlan p;
    p.n = n;
    p.Np = ceil_div(n, kTile) * kTile;
    p.padded = (n % kTile) != 0;
    // a node's n2 x n1 product (T, or U = -Li22 L21) lives from before its
    // leading block's factorisation to its last product, so every depth has
    // its own buffer: an ancestor's stays intact under its descendants
    int64_t most[kFactorDepths] = {0};
    depth_products(p.Np, 0, most);
    int64_t tfloats = 0;
    for (int d = 0; d < kFactorDepths; ++d) {
        p.tbase[d] = tfloats;
        tfloats += most[d];
    }
    size_t off = 0;
    p.off_mean = off;
    off += kAlign;
    p.off_T = off;
    off = align_up(off + sizeof(float) * (size_t)tfloats);
    p.off_L = p.off_P = 0;
    if (p.padded) {
        p.off_L = off;
        off = align_up(off + sizeof(float) * (size_t)(p.Np * p.Np));
        p.off_P = off;
        off = align_up(off + sizeof(float) * (size_t)(p.Np * p.Np));
    }
    p.total = off;
    return p;
}

struct FactorRun {
    float* Lbuf;
    float* Pbuf;
    float* T;                  // the depths' product buffers (tbase)
    const int64_t* tbase;
    int64_t ld;
    int32_t* info;
    hipStream_t s;
    Prof* prof;
    bool early;                // the leading spine finishes its blocks early (see factor_rec)
    const FactorLeads* leads;  // nullable: events of the leading blocks, recorded as they become final
    int64_t n;
    FactorCalls* defer;        // nullable: stream operations are appended here instead of issued
    hipStream_t side;          // the stream of the right-looking pieces (factor_rec); null: s itself
    std::shared_ptr<std::vector<hipEvent_t>> events;   // destroyed with the last operation that holds them
};

int launch_ok() { return hipGetLastError() == hipSuccess ? 0 : -1; }

hipEvent_t new_event(const FactorRun& R)
{
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) return nullptr;
    R.events->push_back(e);
    return e;
}

// One stream operation of the factorisation (f returns 0 or -1): issued at
// once, or appended to R.defer.
template <class F>
int emit(const FactorRun& R, F f)
{
    if (R.defer) {
        R.defer->emplace_back(std::move(f));
        return 0;
    }
    return f();
}

// Records the event of the leading block [0, size)^2 (size below n).
int record_lead(const FactorRun& R, int64_t size)
{
    if (!R.leads) return 0;
    for (int k = 0; k < R.leads->count; ++k)
        if (R.leads->size[k] == size) {
            const hipEvent_t e = R.leads->ev[k];
            const hipStream_t s = R.s;
            return emit(R, [e, s] { return hipEventRecord(e, s) == hipSuccess ? 0 : -1; });
        }
    return 0;
}

// The finish pass over rows [i0, i1) and columns [j0, j1) (multiples of 4):
// P = Li diag(L) below the diagonal, zeros above both diagonals.
int enqueue_finish(const FactorRun& R, int64_t i0, int64_t i1, int64_t j0, int64_t j1)
{
    const double rows = (double)(i1 - i0), cols = (double)(j1 - j0);
    dim3 g((unsigned)ceil_div(j1 - j0, 1024), (unsigned)std::min<int64_t>(i1 - i0, 256));
    return emit(R, [=] {
        launch(R.prof, KK_F_FINISH, rows * cols / 2.0, 4.0 * 4.0 * rows * cols, k_f_finish, g, dim3(256), R.s,
               R.Lbuf, R.Pbuf, R.ld, i0, i1, j0, j1, R.n, (float*)nullptr, (float*)nullptr);
        return launch_ok();
    });
}

// Algorithmic work (fp32 flops = 2 x multiply-adds on the nonzero triangle /
// block support) and bytes (each operand read once, each output written once).
inline double tri(double k) { return k * (k + 1.0) / 2.0; }

// The panel L21 = Li22^T A21 (L21: rows o2 .. o2 + n2 - 1, columns o1 ..
// o1 + n1 - 1) on stream st: 128 x 128 blocks while they fill the GPU, else
// 64 x 64 tiles.
int emit_panel(const FactorRun& R, hipStream_t st, int64_t o1, int64_t o2, int n1, int n2)
{
    const bool tiles = ceil_div(n1, FBN) * ceil_div(n2, FBM) < kFactorBlockMin;
    const dim3 g((unsigned)ceil_div(n1, FBN), (unsigned)ceil_div(n2, FBM));
    const dim3 gt((unsigned)(n1 / kTile), (unsigned)(n2 / kTile));
    const double d1 = n1, d2 = n2;
    const double fl = 2.0 * d1 * tri(d2), by = 4.0 * (tri(d2) + 2.0 * d2 * d1);
    return emit(R, [=] {
        if (tiles)
            launch(R.prof, KK_F_PANEL_T, fl, by, k_f_tile<0>, gt, dim3(256), st, R.Lbuf, R.Pbuf, (float*)nullptr,
                   R.ld, o1, o2, n1, n2, st == R.s ? 1 : 0);
        else
            launch(R.prof, KK_F_PANEL, fl, by, k_f_panel, g, dim3(256), st, R.Pbuf, R.Lbuf, R.ld, o1, o2, n1, n2);
        return launch_ok();
    });
}

// The SYRK A11 -= L21^T L21 on the lower tiles of A11 (o1 .. o1 + n1 - 1),
// L21 rows o2 .. o2 + n2 - 1, on stream st.
int emit_syrk(const FactorRun& R, hipStream_t st, int64_t o1, int64_t o2, int n1, int n2)
{
    const double d1 = n1, d2 = n2;
    const double fl = 2.0 * d2 * tri(d1), by = 4.0 * (d2 * d1 + 2.0 * tri(d1));
    const int64_t tb = n1 / kTile, nsyrk = tb * (tb + 1) / 2;
    return emit(R, [=] {
        launch(R.prof, KK_F_SYRK_T, fl, by, k_f_tile<1>, dim3((unsigned)nsyrk), dim3(256), st, R.Lbuf, R.Pbuf,
               (float*)nullptr, R.ld, o1, o2, n1, n2, st == R.s ? 1 : 0);
        return launch_ok();
    });
}

// A node whose panel and SYRK are split right-looking (see factor_rec)
// passes its leading range to its trailing child, which fills in `done`.
struct Pending {
    int64_t o;          // the node's leading half: columns o .. o + n - 1
    int n;
    hipEvent_t done;    // recorded on the side stream after the child's share
};

#ifndef BAKRON_RIGHT_LOOKING
#define BAKRON_RIGHT_LOOKING 1
#endif
// Tile-level nodes of at least this size (and every block level) are split
// right-looking; such a node forms U = -Li22 L21 on the side stream too.
// (The 7168 halves of a 14336 factor: 0.7-0.9 ms off the fused call at
// 4096 x 14336 and its transpose.  From 4096 down, the two factors of
// separate calls, issued one after the other, queue their side work behind
// each other's on the hardware queue that library slots 2 and 3 share.)
#ifndef BAKRON_RL_MIN
#define BAKRON_RL_MIN 7168
#endif
constexpr int64_t kRLMin = BAKRON_RL_MIN;

// On the leading spine (o == 0, with `early`) every node ends with its
// whole block [0, nsz)^2 finished (P = Li diag(L), zeros above both
// diagonals) and records that block's event: the base block is finished
// after its factorisation; an inner node's two last products use the
// finished P11 and give P21 directly, T' = L21 P11 and
// P21 = Li21 diag(L11) = -Li22 L21 Li11 diag(L11) = -Li22 T', and it then
// finishes its trailing block.  Off the spine the blocks stay unscaled (the
// products of the levels above read Li).
//
// Right-looking split (block levels, with a side stream).  The node's panel
// L21 = Li22^T A21 and SYRK A11 -= L21^T L21 wait for the whole trailing
// half C = [C1 | C2].  But the rows of C2 are final once C2 and C's own panel
// L[C2, C1] are: then, on the side stream, L[C2, A] = Li_C2^T A[C2, A], the
// update A[C1, A] -= L[C2, C1]^T L[C2, A] of the rows still pending, and
// the SYRK share A11 -= L[C2, A]^T L[C2, A] run beside C1's factorisation
// (a chain of small launches).  C1 does the same with its own halves, and
// so on down C's leading spine, so after C only the rows of C's leading-most
// base block are left on the chain: their rows of L21 and their SYRK share.
// The same products in a different grouping (block Gaussian elimination of
// Li_C^T A21 by the blocks of C's leading spine), so the factor's rounding
// changes but not its accuracy.  `up`: the parent's pending columns when
// this node is C or a node of C's leading spine.
int factor_rec(const FactorRun& R, int64_t o, int64_t nsz, int depth, Pending* up)
{
    const bool spine = R.early && o == 0;
    if (nsz <= 2 * kTile) {
        // factor (b^3 / 3 multiply-adds) and inverse (b^3 / 6) of the block
        const double b = (double)nsz;
        if (emit(R, [=] {
                launch(R.prof, KK_F_DIAG, b * b * b, 4.0 * (tri(b) + 2.0 * b * b), k_f_diag, dim3(1), dim3(kDiagThreads), R.s,
                       R.Lbuf, R.Pbuf, R.ld, o, (int)nsz, R.info);
                return launch_ok();
            }))
            return -1;
        if (spine && (enqueue_finish(R, 0, nsz, 0, nsz) || record_lead(R, nsz))) return -1;
        return 0;
    }
    const int64_t nt = nsz / kTile;
    const int n1 = (int)(kTile * (nt / 2));
    const int n2 = (int)(nsz - n1);
    const int64_t o1 = o, o2 = o + n1;
    const double d1 = n1, d2 = n2;
    if (depth >= kFactorDepths) return -1;
    float* const T = R.T + R.tbase[depth];
    // 128 x 128 blocks while they fill the GPU, else 64 x 64 tiles
    const bool tiles = ceil_div(n1, FBN) * ceil_div(n2, FBM) < kFactorBlockMin;
    const dim3 g((unsigned)ceil_div(n1, FBN), (unsigned)ceil_div(n2, FBM));
    const dim3 gt((unsigned)(n1 / kTile), (unsigned)(n2 / kTile));
    const bool rl = BAKRON_RIGHT_LOOKING && (!tiles || nsz >= kRLMin) && n2 > 2 * kTile;
    hipEvent_t u_done = nullptr;   // a right-looking tile-level node forms U on the side stream
    // This node as the trailing half of a right-looking parent (`up`): once
    // its own panel is formed, its rows o2 .. o2 + n2 - 1 are final for the
    // parent's columns too.  On the side stream: those rows of the parent's
    // panel, the update of this node's rows o1 .. o2 - 1 for the parent's
    // columns, and the parent's SYRK share of the final rows.
    auto parent_share = [&]() -> int {
        if (!up) return 0;
        const hipEvent_t ready = new_event(R), done = new_event(R);
        if (!ready || !done) return -1;
        const hipStream_t s = R.s, side = R.side ? R.side : R.s;
        const int64_t po = up->o;
        const int pn = up->n;
        const double fu = 2.0 * d1 * pn * d2, bu = 4.0 * (2.0 * d1 * pn + d2 * (d1 + pn));
        const dim3 gu((unsigned)ceil_div(pn, FBN), (unsigned)ceil_div(n1, FBM));
        if (emit(R, [=] {
                return (hipEventRecord(ready, s) == hipSuccess && hipStreamWaitEvent(side, ready, 0) == hipSuccess)
                           ? 0
                           : -1;
            }) ||
            emit_panel(R, side, po, o2, pn, n2) ||
            emit(R, [=] {
                launch(R.prof, KK_F_UPDATE, fu, bu, k_f_update, gu, dim3(256), side, (const float*)R.Lbuf, R.Pbuf,
                       R.ld, o1, po, o2, n1, pn, n2);
                return launch_ok();
            }) ||
            emit_syrk(R, side, po, o2, pn, n2) ||
            emit(R, [=] { return hipEventRecord(done, side) == hipSuccess ? 0 : -1; }))
            return -1;
        up->done = done;
        return 0;
    };
    Pending mine{o1, n1, nullptr};
    if (factor_rec(R, o2, n2, depth + 1, rl ? &mine : nullptr)) return -1;
    if (rl) {
        // the side stream's share (rows of C2) is done; the rows of C1 here
        const hipEvent_t e = mine.done;
        const hipStream_t s = R.s;
        if (!e || emit(R, [=] { return hipStreamWaitEvent(s, e, 0) == hipSuccess ? 0 : -1; })) return -1;
        int c1 = n2;   // the rows left: C's leading-most base block
        while (c1 > 2 * kTile) c1 = (int)(kTile * ((c1 / kTile) / 2));
        if (emit_panel(R, R.s, o1, o2, n1, c1) || parent_share()) return -1;
        if (tiles) {
            // U = -Li22 L21 (L21 is complete now) on the side stream, beside
            // the leading half's factorisation; Li21 = U Li11 waits for it
            const hipEvent_t ready = new_event(R);
            u_done = new_event(R);
            if (!ready || !u_done) return -1;
            const hipStream_t side = R.side ? R.side : R.s;
            const double fu = 2.0 * d1 * tri(d2), bu = 4.0 * (2.0 * d2 * d1 + tri(d2));
            const hipEvent_t ud = u_done;
            if (emit(R, [=] {
                    return (hipEventRecord(ready, s) == hipSuccess && hipStreamWaitEvent(side, ready, 0) == hipSuccess)
                               ? 0
                               : -1;
                }) ||
                emit(R, [=] {
                    launch(R.prof, KK_F_U_T, fu, bu, k_f_tile<4>, dim3(gt.x * gt.y), dim3(256), side, R.Lbuf,
                           R.Pbuf, T, R.ld, o1, o2, n1, n2, side == R.s ? 1 : 0);
                    return launch_ok();
                }) ||
                emit(R, [=] { return hipEventRecord(ud, side) == hipSuccess ? 0 : -1; }))
                return -1;
        }
        if (emit_syrk(R, R.s, o1, o2, n1, c1)) return -1;
    } else {
        if (emit_panel(R, R.s, o1, o2, n1, n2) || parent_share()) return -1;
        if (tiles) {
            // SYRK on 64 x 64 tiles at every level: its K extent is uniform, so
            // the finer grid only helps (a triangle of 128-blocks quantizes badly
            // over the CUs, e.g. 528 blocks at n1 = 4096).  On the tile levels
            // the same launch forms U = -Li22 L21.
            const double fl = 2.0 * d2 * tri(d1), by = 4.0 * (d2 * d1 + 2.0 * tri(d1));
            const double fu = 2.0 * d1 * tri(d2), bu = 4.0 * (2.0 * d2 * d1 + tri(d2));
            const int64_t tb = n1 / kTile, nsyrk = tb * (tb + 1) / 2;
            if (emit(R, [=] {
                    launch(R.prof, KK_F_LEFT_T, fl + fu, by + bu, k_f_tile<3>, dim3((unsigned)(nsyrk + gt.x * gt.y)),
                           dim3(256), R.s, R.Lbuf, R.Pbuf, T, R.ld, o1, o2, n1, n2, 1);
                    return launch_ok();
                }))
                return -1;
        } else if (emit_syrk(R, R.s, o1, o2, n1, n2)) {
            return -1;
        }
    }
    // the parent's pending rows continue down the leading half (its trailing
    // rows go to the side stream there too), so that only this node's
    // leading-most base block is left for the parent's chain
    if (factor_rec(R, o1, n1, depth + 1, n1 > 2 * kTile ? up : nullptr)) return -1;
    {
        const double fr = 2.0 * d2 * tri(d1), br = 4.0 * (2.0 * d2 * d1 + tri(d1));
        const double fl = 2.0 * d1 * tri(d2), bl = 4.0 * (2.0 * d2 * d1 + tri(d2));
        if (tiles) {
            // Li21 = U Li11 (on the spine U P11 = P21, P11 being finished)
            if (u_done) {
                const hipEvent_t e = u_done;
                const hipStream_t s = R.s;
                if (emit(R, [=] { return hipStreamWaitEvent(s, e, 0) == hipSuccess ? 0 : -1; })) return -1;
            }
            if (emit(R, [=] {
                    launch(R.prof, KK_F_RIGHT_T, fr, br, k_f_tile<2>, dim3(gt.y, gt.x), dim3(256), R.s, R.Lbuf,
                           R.Pbuf, T, R.ld, o1, o2, n1, n2, 1);
                    return launch_ok();
                }))
                return -1;
        } else if (R.leads && o == 0 && nsz == R.ld && (g.x * g.y <= kLeadMaxBlocks || kLeadGridBig > 0)) {
            static std::once_flag attrs;
            std::call_once(attrs, [] {
                (void)hipFuncSetAttribute((const void*)k_f_right_lead, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)kLeadPad);
                (void)hipFuncSetAttribute((const void*)k_f_left_lead, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)kLeadPad);
            });
            const unsigned cnt = g.x * g.y, grid = std::min(cnt, cnt <= kLeadMaxBlocks ? kLeadGrid : kLeadGridBig);
            if (emit(R, [=] {
                    launch_shm(R.prof, KK_F_RIGHT, fr, br, k_f_right_lead, dim3(grid), dim3(256), kLeadPad, R.s,
                               (const float*)R.Lbuf, (const float*)R.Pbuf, T, R.ld, o1, o2, n1, n2, g.y, cnt);
                    launch_shm(R.prof, KK_F_LEFT, fl, bl, k_f_left_lead, dim3(grid), dim3(256), kLeadPad, R.s,
                               (const float*)T, R.Pbuf, R.ld, o1, o2, n1, n2, g.x, g.y, cnt);
                    return launch_ok();
                }))
                return -1;
        } else {
            if (emit(R, [=] {
                    launch(R.prof, KK_F_RIGHT, fr, br, k_f_right, dim3(g.y, g.x), dim3(256), R.s,
                           (const float*)R.Lbuf, (const float*)R.Pbuf, T, R.ld, o1, o2, n1, n2);
                    launch(R.prof, KK_F_LEFT, fl, bl, k_f_left, g, dim3(256), R.s, (const float*)T, R.Pbuf, R.ld, o1,
                           o2, n1, n2);
                    return launch_ok();
                }))
                return -1;
        }
    }
    if (spine) {   // the trailing block, and the zeros right of the leading block (P21 is done)
        if (enqueue_finish(R, n1, nsz, n1, nsz) || enqueue_finish(R, 0, n1, n1, nsz) ||
            (nsz < R.ld && record_lead(R, nsz)))
            return -1;
    }
    return 0;
}

}  // namespace

size_t factor_workspace_bytes(int64_t n)
{
    if (n <= 0) return 0;
    return plan_factor(n).total;
}

int factor_leads(int64_t n, int64_t* sizes)
{
    if (n <= 2 * kTile || n % kTile != 0) return 0;
    int count = 0;
    int64_t spine[kMaxLeads];
    for (int64_t sz = n; sz > 2 * kTile && count < kMaxLeads;) {
        sz = kTile * (sz / kTile / 2);
        spine[count++] = sz;
    }
    for (int k = 0; k < count; ++k) sizes[k] = spine[count - 1 - k];   // smallest first
    return count;
}

int factor_enqueue(const float* A, int64_t n, float damp_frac, float* L, float* P, int32_t* info,
                   void* ws, hipStream_t s, Prof* prof, const FactorLeads* leads, FactorCalls* defer,
                   hipStream_t side)
{
    const FactorPlan p = plan_factor(n);
    char* w = static_cast<char*>(ws);
    float* mean = reinterpret_cast<float*>(w + p.off_mean);
    FactorRun R;
    R.T = reinterpret_cast<float*>(w + p.off_T);
    R.tbase = p.tbase;
    R.ld = p.Np;
    R.info = info;
    R.s = s;
    R.prof = prof;
    int64_t sizes[kMaxLeads];
    R.early = factor_leads(n, sizes) > 0;
    R.leads = R.early ? leads : nullptr;
    R.n = n;
    R.Lbuf = p.padded ? reinterpret_cast<float*>(w + p.off_L) : L;
    R.Pbuf = p.padded ? reinterpret_cast<float*>(w + p.off_P) : P;
    R.defer = defer;
    R.side = side;
    R.events = std::shared_ptr<std::vector<hipEvent_t>>(new std::vector<hipEvent_t>(), [](std::vector<hipEvent_t>* v) {
        for (hipEvent_t e : *v) (void)hipEventDestroy(e);
        delete v;
    });
    const double dn = (double)n, dN = (double)p.Np;
    const int64_t Np = p.Np;
    float* const Lb = R.Lbuf;
    float* const Pb = R.Pbuf;

    {
        dim3 g((unsigned)ceil_div(Np, 1024), (unsigned)std::min<int64_t>(Np, 32768));
        const int vec = (n % 4 == 0 && aligned16(A)) ? 1 : 0;
        if (emit(R, [=] {
                launch(prof, KK_F_CLEAR, 0.0, 4.0, k_clear_info, dim3(1), dim3(64), s, info);
                launch(prof, KK_F_MEAN, 0.0, 4.0 * dn, k_diag_mean, dim3(1), dim3(256), s, A, n, mean);
                launch(prof, KK_F_LOAD, dn, 4.0 * (tri(dn) + dN * dN), k_load_damped, g, dim3(256), s, A, n, Pb, Np,
                       Np, (const float*)mean, damp_frac, vec);
                return launch_ok();
            }))
            return -1;
    }
    if (factor_rec(R, 0, Np, 0, nullptr)) return -1;
    if (defer) {   // the events live until the deferred list is destroyed
        auto keep = R.events;
        defer->emplace_back([keep] { return 0; });
    }
    if (!R.early) {   // (on the early path every block of the spine has been finished)
        dim3 g((unsigned)ceil_div(Np, 1024), (unsigned)std::min<int64_t>(Np, 256));
        float* const Lo = p.padded ? L : nullptr;
        float* const Po = p.padded ? P : nullptr;
        return emit(R, [=] {
            launch(prof, KK_F_FINISH, dn * dn / 2.0, 4.0 * (2.0 * tri(dN) + 2.0 * dn * dn), k_f_finish, g,
                   dim3(256), s, Lb, Pb, Np, (int64_t)0, Np, (int64_t)0, Np, n, Lo, Po);
            return launch_ok();
        });
    }
    return 0;
}

int run_interleaved(FactorCalls& a, FactorCalls& b)
{
    const size_t n = std::max(a.size(), b.size());
    for (size_t i = 0; i < n; ++i) {
        if (i < a.size() && a[i]()) return -1;
        if (i < b.size() && b[i]()) return -1;
    }
    return 0;
}

}  // namespace bk
