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
// recurse on 1; Li21 = -Li22 (L21 Li11) (two GEMMs).  Diagonal blocks of 128
// (or 64) are factored and inverted in LDS by one workgroup.
//
// Buffers: Pbuf starts as A_d (lower part used) and ends as Li; Lbuf
// receives L.  Both are n x n with pitch ld.  The temporary T (n2 x n1) lives
// in the workspace.  A final pass scales Li's columns by diag(L) (giving P)
// and writes zeros above both diagonals.
#include <algorithm>

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
__global__ __launch_bounds__(256) void k_load_damped(const float* __restrict__ A, int64_t n,
                                                     float* __restrict__ dst, int64_t Np, int64_t ld,
                                                     const float* __restrict__ mean, float frac)
{
    // frac == 0 adds nothing (not 0 * mean, which is NaN for a non-finite diagonal)
    const float add = frac != 0.f ? frac * mean[0] : 0.f;
    for (int64_t i = blockIdx.y; i < Np; i += gridDim.y)
        for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < Np; j += (int64_t)gridDim.x * 256) {
            float v = 0.f;
            if (i < n && j < n) {
                if (j < i) v = A[i * n + j];
                else if (j == i) v = A[i * n + j] + add;
            } else if (i == j) {
                v = 1.f;
            }
            dst[i * ld + j] = v;
        }
}

// --------------------------------------------------- diagonal blocks
//
// k_f_diag factors a whole diagonal block of 64 or 128 in one workgroup,
// with the block and its inverse resident in LDS (2 x 128 x 132 floats):
//   size 64:  base64 (reverse Cholesky and inverse) of the block;
//   size 128: base64 of the trailing 64 (L22, Li22); L21 = Li22^T A21;
//             A11 -= L21^T L21; base64 of A11 (L11, Li11);
//             Li21 = -Li22 (L21 Li11)
// -- the same recursion as the GEMM levels above it, with the four 64^3
// products on the MFMA units straight from LDS.

constexpr int kDP = 132;   // LDS pitch (floats) of the block and its inverse

// base64: reverse Cholesky S = L^T L of the 64 x 64 block at S (pitch kDP,
// lower part read), then X = L^-1; L overwrites S and X goes to X (both with
// zeros above the diagonal).  256 threads: thread t owns row i = t / 4,
// columns 16 (t % 4) .. + 15, in registers.
//
// Elimination from the last row up, on unscaled rows: at step k every row
// i < k takes S[i][j] -= (S[k][i] / S[k][k]) S[k][j]; row k is read from a
// double-buffered LDS row that its owners published at the end of the
// previous step, so a step costs one barrier.  At the end each row is scaled
// once, L[i][j] = S[i][j] / sqrt(S[i][i]) (S[i][i] taken when row i was the
// pivot).  The inverse solves L X = I by rows, forward: with
// R[i] = L[i][i] X[i], R[i] = e_i - sum_{k<i} (L[i][k] / L[k][k]) R[k], the
// same one-row-per-step broadcast.  Reciprocals and square roots use the
// hardware approximations (about one ulp): the factor is judged by its
// backward error, not by correct rounding.
//
// Returns the block row of the first non-positive (or NaN) pivot met, or -1.
__device__ __forceinline__ int base64(float* __restrict__ S, float* __restrict__ X, float* __restrict__ rowbuf)
{
    const int t = threadIdx.x;
    const int i = t >> 2, c0 = 16 * (t & 3);
    float s[16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(S + i * kDP + c0 + 4 * u);
        s[4 * u + 0] = v.x;
        s[4 * u + 1] = v.y;
        s[4 * u + 2] = v.z;
        s[4 * u + 3] = v.w;
    }
    if (i == 63)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<f32x4*>(rowbuf + 64 + c0 + 4 * u) =
                f32x4{s[4 * u], s[4 * u + 1], s[4 * u + 2], s[4 * u + 3]};
    __syncthreads();
    int fail = -1;
    float mypiv = 1.f;
    // One elimination step with pivot row k in rk; row k - 1 goes to rnext.
    auto chol_step = [&](const int k, const float* rk, float* rnext) {
        const float piv = rk[k];
        const float ski = rk[i];                          // S[k][i] = S[i][k]
        f32x4 r[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = *reinterpret_cast<const f32x4*>(rk + c0 + 4 * u);
        if (!(piv > 0.f) && fail < 0) fail = k;
        if (i == k) mypiv = piv;
        const float mul = (i < k) ? ski * __builtin_amdgcn_rcpf(piv) : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            s[4 * u + 0] = fmaf(-mul, r[u].x, s[4 * u + 0]);
            s[4 * u + 1] = fmaf(-mul, r[u].y, s[4 * u + 1]);
            s[4 * u + 2] = fmaf(-mul, r[u].z, s[4 * u + 2]);
            s[4 * u + 3] = fmaf(-mul, r[u].w, s[4 * u + 3]);
        }
        if (i == k - 1)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<f32x4*>(rnext + c0 + 4 * u) =
                    f32x4{s[4 * u], s[4 * u + 1], s[4 * u + 2], s[4 * u + 3]};
        __syncthreads();
    };
    // The step loops stay loops (two steps per iteration, for the buffer
    // parity): a fully unrolled base is thousands of straight-line
    // instructions that run once each, and their fetch would dominate.
#pragma unroll 1
    for (int k = 63; k > 0; k -= 2) {
        chol_step(k, rowbuf + 64, rowbuf);
        chol_step(k - 1, rowbuf, rowbuf + 64);
    }
    const float rs = __builtin_amdgcn_rsqf(mypiv);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4 v;
        v.x = (c0 + 4 * u + 0 <= i) ? s[4 * u + 0] * rs : 0.f;
        v.y = (c0 + 4 * u + 1 <= i) ? s[4 * u + 1] * rs : 0.f;
        v.z = (c0 + 4 * u + 2 <= i) ? s[4 * u + 2] * rs : 0.f;
        v.w = (c0 + 4 * u + 3 <= i) ? s[4 * u + 3] * rs : 0.f;
        *reinterpret_cast<f32x4*>(S + i * kDP + c0 + 4 * u) = v;
    }
    // R = I; row 0 published
    float r[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) r[c] = (c0 + c == i) ? 1.f : 0.f;
    if (i == 0)
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<f32x4*>(rowbuf + c0 + 4 * u) = f32x4{r[4 * u], r[4 * u + 1], r[4 * u + 2], r[4 * u + 3]};
    __syncthreads();
    // One substitution step with R[k] in rk; R[k + 1] goes to rnext (k = 63
    // is a no-op that keeps the trip count even).
    auto inv_step = [&](const int k, const float* rk, float* rnext) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4*>(rk + c0 + 4 * u);
        const float coef = (i > k) ? S[i * kDP + k] * __builtin_amdgcn_rcpf(S[k * kDP + k]) : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            r[4 * u + 0] = fmaf(-coef, v[u].x, r[4 * u + 0]);
            r[4 * u + 1] = fmaf(-coef, v[u].y, r[4 * u + 1]);
            r[4 * u + 2] = fmaf(-coef, v[u].z, r[4 * u + 2]);
            r[4 * u + 3] = fmaf(-coef, v[u].w, r[4 * u + 3]);
        }
        if (i == k + 1)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                *reinterpret_cast<f32x4*>(rnext + c0 + 4 * u) =
                    f32x4{r[4 * u], r[4 * u + 1], r[4 * u + 2], r[4 * u + 3]};
        __syncthreads();
    };
#pragma unroll 1
    for (int k = 0; k < 64; k += 2) {
        inv_step(k, rowbuf, rowbuf + 64);
        inv_step(k + 1, rowbuf + 64, rowbuf);
    }
    const float inv = __builtin_amdgcn_rcpf(S[i * kDP + i]);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        f32x4 v;
        v.x = (c0 + 4 * u + 0 <= i) ? r[4 * u + 0] * inv : 0.f;
        v.y = (c0 + 4 * u + 1 <= i) ? r[4 * u + 1] * inv : 0.f;
        v.z = (c0 + 4 * u + 2 <= i) ? r[4 * u + 2] * inv : 0.f;
        v.w = (c0 + 4 * u + 3 <= i) ? r[4 * u + 3] * inv : 0.f;
        *reinterpret_cast<f32x4*>(X + i * kDP + c0 + 4 * u) = v;
    }
    __syncthreads();
    return fail;
}

// MFMA fragment of LDS operand element (r, k .. k + 3) (pitch kDP):
// RowK p[r * kDP + k], KRow p[k * kDP + r].
template <int LAYOUT>
__device__ __forceinline__ f32x4 ldsfrag(const float* p, int r, int k)
{
    if (LAYOUT == RowK) return *reinterpret_cast<const f32x4*>(p + r * kDP + k);
    return f32x4{p[k * kDP + r], p[(k + 1) * kDP + r], p[(k + 2) * kDP + r], p[(k + 3) * kDP + r]};
}

// 64 x 64 x 64 product from LDS: wave w returns the 32 x 32 quadrant at rows
// 32 (w >> 1), columns 32 (w & 1) of A B, with A(r, k) and B(k, c) addressed
// as ldsfrag's (r, k) and (c, k).
template <int ALAY, int BLAY>
__device__ __forceinline__ f32x16 lds_mm64(const float* A, const float* B)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ml = lane & 31, k4 = 4 * (lane >> 5);
    const int ra = 32 * (wave >> 1) + ml, rb = 32 * (wave & 1) + ml;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 64; kc += 8) {
        const f32x4 a = ldsfrag<ALAY>(A, ra, kc + k4);
        const f32x4 b = ldsfrag<BLAY>(B, rb, kc + k4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
    }
    return acc;
}

// C (64 x 64 in LDS) = alpha * acc + beta * C over this wave's quadrant.
__device__ __forceinline__ void lds_put64(float* C, const f32x16& acc, float alpha, float beta)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = 32 * (wave & 1) + (lane & 31);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 32 * (wave >> 1) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        float* p = C + row * kDP + col;
        *p = alpha * acc[r] + (beta != 0.f ? beta * *p : 0.f);
    }
}

__global__ __launch_bounds__(256) void k_f_diag(float* __restrict__ Lbuf, float* __restrict__ Pbuf, int64_t ld,
                                                int64_t o, int nb, int32_t* __restrict__ info)
{
    __shared__ __align__(16) float sA[128 * kDP];   // the block, then L
    __shared__ __align__(16) float sX[128 * kDP];   // L^-1
    __shared__ __align__(16) float rowbuf[128];
    const int t = threadIdx.x;
    const int nf4 = nb / 4;
    for (int f = t; f < nb * nf4; f += 256) {
        const int r = f / nf4, c = 4 * (f % nf4);
        *reinterpret_cast<f32x4*>(sA + r * kDP + c) =
            *reinterpret_cast<const f32x4*>(Pbuf + (o + r) * ld + o + c);
    }
    __syncthreads();
    // pass 1 (size 128 only): trailing half and the products it feeds;
    // pass 0: the leading half (or the whole size-64 block) and, for 128,
    // the off-diagonal block of the inverse.  One inlined copy of base64.
    int fail[2] = {-1, -1};
    float* A21 = sA + 64 * kDP;
    float* X22 = sX + 64 * kDP + 64;
    for (int h = (nb == 128) ? 1 : 0; h >= 0; --h) {
        fail[h] = base64(sA + h * (64 * kDP + 64), sX + h * (64 * kDP + 64), rowbuf);
        if (nb != 128) break;
        if (h == 1) {
            f32x16 acc = lds_mm64<KRow, KRow>(X22, A21);          // L21 = Li22^T A21
            __syncthreads();
            lds_put64(A21, acc, 1.f, 0.f);
            __syncthreads();
            acc = lds_mm64<KRow, KRow>(A21, A21);                 // A11 -= L21^T L21
            lds_put64(sA, acc, -1.f, 1.f);
            __syncthreads();
        } else {
            f32x16 acc = lds_mm64<RowK, KRow>(A21, sX);           // T = L21 Li11 (into X's upper block)
            lds_put64(sX + 64, acc, 1.f, 0.f);
            __syncthreads();
            acc = lds_mm64<RowK, KRow>(X22, sX + 64);             // Li21 = -Li22 T
            lds_put64(sX + 64 * kDP, acc, -1.f, 0.f);
            __syncthreads();
        }
    }
    for (int f = t; f < nb * nf4; f += 256) {
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
    if (t == 0) {   // the trailing half is factored first: its failure is met first
        if (fail[1] >= 0) atomicCAS(info, 0, (int32_t)(o + 64 + fail[1] + 1));
        if (fail[0] >= 0) atomicCAS(info, 0, (int32_t)(o + fail[0] + 1));
    }
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

// The same four products with one 64 x 64 output tile per workgroup (one
// 32 x 32 quadrant per wave) for the levels whose 128 x 128 grids are too
// small to fill the GPU.  MODE: 0 panel, 1 syrk, 2 right, 3 left.
template <int MODE>
__global__ __launch_bounds__(256) void k_f_tile(float* __restrict__ Lbuf, float* __restrict__ Pbuf,
                                                float* __restrict__ T, int64_t ld, int64_t o1, int64_t o2,
                                                int n1, int n2)
{
    __shared__ __align__(16) float lds[kLds64];
    int r0, c0;
    if (MODE == 1) {   // linear index -> lower-triangular tile (br >= bc)
        const int q = blockIdx.x;
        int br = (int)((sqrtf(8.f * q + 1.f) - 1.f) * 0.5f);
        while ((br + 1) * (br + 2) / 2 <= q) ++br;
        while (br * (br + 1) / 2 > q) --br;
        r0 = 64 * br;
        c0 = 64 * (q - br * (br + 1) / 2);
    } else if (MODE == 3) {   // heaviest (largest K) first
        r0 = 64 * (int)(gridDim.y - 1 - blockIdx.y);
        c0 = 64 * (int)blockIdx.x;
    } else if (MODE == 2) {   // rows along x: the longest column tiles first
        r0 = 64 * (int)blockIdx.x;
        c0 = 64 * (int)blockIdx.y;
    } else {
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
    } else if (MODE == 1) {   // A11 -= L21^T L21, lower part
        block_gemm64<KRow, KRow>(Lbuf + o2 * ld + o1 + r0, ld, Lbuf + o2 * ld + o1 + c0, ld, 0, n2, lds, acc);
        wave_store32(Pbuf + (o1 + r0 + qr) * ld + o1 + c0 + qc, ld, -1.f, 1.f, acc, (c0 + qc) - (r0 + qr));
    } else if (MODE == 2) {   // T = L21 Li11, K in [c0, n1)
        block_gemm64<RowK, KRow>(Lbuf + (o2 + r0) * ld + o1, ld, Pbuf + o1 * ld + o1 + c0, ld, c0, n1, lds, acc);
        wave_store32(T + (int64_t)(r0 + qr) * n1 + c0 + qc, n1, 1.f, 0.f, acc);
    } else {                  // Li21 = -Li22 T, K in [0, r0 + 64)
        block_gemm64<RowK, KRow>(Pbuf + (o2 + r0) * ld + o2, ld, T + c0, n1, 0, r0 + 64, lds, acc);
        wave_store32(Pbuf + (o2 + r0 + qr) * ld + o1 + c0 + qc, ld, -1.f, 0.f, acc);
    }
}

// P = Li diag(L) on and below the diagonal, zeros above, for L and P; when
// the factor ran in padded workspace, also copy the leading n x n out.
// Each thread owns four adjacent columns for a stripe of rows, so the
// diagonal entries it scales by are read once.
__global__ __launch_bounds__(256) void k_f_finish(float* __restrict__ Lbuf, float* __restrict__ Pbuf, int64_t ld,
                                                  int64_t Np, int64_t n, float* __restrict__ Lout,
                                                  float* __restrict__ Pout)
{
    const int64_t j = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x);
    if (j >= Np) return;
    float dg[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) dg[q] = Lbuf[(j + q) * ld + j + q];
    for (int64_t i = blockIdx.y; i < Np; i += gridDim.y) {
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

struct FactorPlan {
    int64_t n, Np;
    bool padded;
    size_t off_mean, off_T, off_L, off_P, total;
};

FactorPlan plan_factor(int64_t n)
{
    FactorPlan p;
    p.n = n;
    p.Np = ceil_div(n, kTile) * kTile;
    p.padded = (n % kTile) != 0;
    const int64_t nt = p.Np / kTile;
    const int64_t n1 = kTile * (nt / 2), n2 = p.Np - n1;
    size_t off = 0;
    p.off_mean = off;
    off += kAlign;
    p.off_T = off;
    off = align_up(off + sizeof(float) * (size_t)(n1 * n2));
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
    float* T;
    int64_t ld;
    int32_t* info;
    hipStream_t s;
    Prof* prof;
};

// Algorithmic work (fp32 flops = 2 x multiply-adds on the nonzero triangle /
// block support) and bytes (each operand read once, each output written once).
inline double tri(double k) { return k * (k + 1.0) / 2.0; }

int launch_ok() { return hipGetLastError() == hipSuccess ? 0 : -1; }

int factor_rec(const FactorRun& R, int64_t o, int64_t nsz)
{
    if (nsz <= 2 * kTile) {
        // factor (b^3 / 3 multiply-adds) and inverse (b^3 / 6) of the block
        const double b = (double)nsz;
        launch(R.prof, KK_F_DIAG, b * b * b, 4.0 * (tri(b) + 2.0 * b * b), k_f_diag, dim3(1), dim3(256), R.s,
               R.Lbuf, R.Pbuf, R.ld, o, (int)nsz, R.info);
        return launch_ok();
    }
    const int64_t nt = nsz / kTile;
    const int n1 = (int)(kTile * (nt / 2));
    const int n2 = (int)(nsz - n1);
    const int64_t o1 = o, o2 = o + n1;
    const double d1 = n1, d2 = n2;
    if (factor_rec(R, o2, n2)) return -1;
    // 128 x 128 blocks while they fill the GPU, else 64 x 64 tiles
    const bool tiles = ceil_div(n1, FBN) * ceil_div(n2, FBM) < kFactorBlockMin;
    const dim3 g((unsigned)ceil_div(n1, FBN), (unsigned)ceil_div(n2, FBM));
    const dim3 gt((unsigned)(n1 / kTile), (unsigned)(n2 / kTile));
    const double fl_panel = 2.0 * d1 * tri(d2), by_panel = 4.0 * (tri(d2) + 2.0 * d2 * d1);
    if (tiles)
        launch(R.prof, KK_F_PANEL_T, fl_panel, by_panel, k_f_tile<0>, gt, dim3(256), R.s, R.Lbuf, R.Pbuf,
               R.T, R.ld, o1, o2, n1, n2);
    else
        launch(R.prof, KK_F_PANEL, fl_panel, by_panel, k_f_panel, g, dim3(256), R.s, R.Pbuf, R.Lbuf, R.ld, o1, o2,
               n1, n2);
    {
        // SYRK on 64 x 64 tiles at every level: its K extent is uniform, so
        // the finer grid only helps (a triangle of 128-blocks quantizes badly
        // over the CUs, e.g. 528 blocks at n1 = 4096).
        const double fl = 2.0 * d2 * tri(d1), by = 4.0 * (d2 * d1 + 2.0 * tri(d1));
        const int64_t tb = n1 / kTile;
        launch(R.prof, KK_F_SYRK_T, fl, by, k_f_tile<1>, dim3((unsigned)(tb * (tb + 1) / 2)), dim3(256), R.s, R.Lbuf,
               R.Pbuf, R.T, R.ld, o1, o2, n1, n2);
    }
    if (launch_ok()) return -1;
    if (factor_rec(R, o1, n1)) return -1;
    {
        const double fr = 2.0 * d2 * tri(d1), br = 4.0 * (2.0 * d2 * d1 + tri(d1));
        const double fl = 2.0 * d1 * tri(d2), bl = 4.0 * (2.0 * d2 * d1 + tri(d2));
        if (tiles) {
            launch(R.prof, KK_F_RIGHT_T, fr, br, k_f_tile<2>, dim3(gt.y, gt.x), dim3(256), R.s, R.Lbuf, R.Pbuf, R.T,
                   R.ld, o1, o2, n1, n2);
            launch(R.prof, KK_F_LEFT_T, fl, bl, k_f_tile<3>, gt, dim3(256), R.s, R.Lbuf, R.Pbuf, R.T,
                   R.ld, o1, o2, n1, n2);
        } else {
            launch(R.prof, KK_F_RIGHT, fr, br, k_f_right, dim3(g.y, g.x), dim3(256), R.s, (const float*)R.Lbuf,
                   (const float*)R.Pbuf, R.T, R.ld, o1, o2, n1, n2);
            launch(R.prof, KK_F_LEFT, fl, bl, k_f_left, g, dim3(256), R.s, (const float*)R.T, R.Pbuf, R.ld, o1, o2,
                   n1, n2);
        }
    }
    return launch_ok();
}

}  // namespace

size_t factor_workspace_bytes(int64_t n)
{
    if (n <= 0) return 0;
    return plan_factor(n).total;
}

int factor_enqueue(const float* A, int64_t n, float damp_frac, float* L, float* P, int32_t* info,
                   void* ws, hipStream_t s, Prof* prof)
{
    const FactorPlan p = plan_factor(n);
    char* w = static_cast<char*>(ws);
    float* mean = reinterpret_cast<float*>(w + p.off_mean);
    FactorRun R;
    R.T = reinterpret_cast<float*>(w + p.off_T);
    R.ld = p.Np;
    R.info = info;
    R.s = s;
    R.prof = prof;
    R.Lbuf = p.padded ? reinterpret_cast<float*>(w + p.off_L) : L;
    R.Pbuf = p.padded ? reinterpret_cast<float*>(w + p.off_P) : P;
    const double dn = (double)n, dN = (double)p.Np;

    launch(prof, KK_F_CLEAR, 0.0, 4.0, k_clear_info, dim3(1), dim3(64), s, info);
    launch(prof, KK_F_MEAN, 0.0, 4.0 * dn, k_diag_mean, dim3(1), dim3(256), s, A, n, mean);
    {
        dim3 g((unsigned)ceil_div(p.Np, 256), (unsigned)std::min<int64_t>(p.Np, 32768));
        launch(prof, KK_F_LOAD, dn, 4.0 * (tri(dn) + dN * dN), k_load_damped, g, dim3(256), s, A, n, R.Pbuf,
               p.Np, p.Np, (const float*)mean, damp_frac);
    }
    if (launch_ok()) return -1;
    if (factor_rec(R, 0, p.Np)) return -1;
    {
        dim3 g((unsigned)ceil_div(p.Np, 1024), (unsigned)std::min<int64_t>(p.Np, 256));
        launch(prof, KK_F_FINISH, dn * dn / 2.0, 4.0 * (2.0 * tri(dN) + 2.0 * dn * dn), k_f_finish, g, dim3(256),
               s, R.Lbuf, R.Pbuf, p.Np, p.Np, n, p.padded ? L : (float*)nullptr, p.padded ? P : (float*)nullptr);
    }
    return launch_ok();
}

}  // namespace bk
