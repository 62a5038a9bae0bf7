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
// recurse on 1; Li21 = -Li22 (L21 Li11) (two GEMMs).  64 x 64 diagonal blocks
// are factored and inverted in LDS by one workgroup.  Total 2n^3/3 flops.
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

// ------------------------------------------------- 64 x 64 diagonal block

// Reverse Cholesky of the 64 x 64 block at offset o of Pbuf (lower part
// read), then its inverse; writes L to Lbuf and L^-1 to Pbuf (zeros above the
// diagonal).  A non-positive (or NaN) pivot at block row k records
// info = o + k + 1 unless an earlier block already recorded one.
//
// One wave; lane i keeps row i of the (symmetric) working block in
// registers, and every loop is unrolled so register indices are constants.
// Elimination from the last row upward: at step k lane k publishes row k in
// LDS, every lane reads it back with 16-byte broadcast loads, lane i (< k)
// takes its multiplier S[i][k] / S[k][k] from its own register k (symmetry)
// and updates its row.  The rows stay unscaled during the elimination; each
// lane scales its own row once at the end, L[i][j] = S[i][j] / sqrt(S[i][i]).
// Then the inverse X = L^-1 row by row from X L = I: lane i computes
// X[i][j] = -(sum_{k=j+1..i} X[i][k] L[k][j]) / L[j][j] for j = i-1 .. 0, all
// rows in parallel, reading column j of L from LDS.  Reciprocals and square
// roots use the hardware approximations (about one ulp): the factor is
// judged by its backward error, not by correct rounding.
__global__ __launch_bounds__(64) void k_base_block(float* __restrict__ Lbuf, float* __restrict__ Pbuf,
                                                   int64_t ld, int64_t o, int32_t* __restrict__ info)
{
    __shared__ __align__(16) float sT[64 * 68];      // staging, then L^T (sT[j][k] = L[k][j])
    __shared__ __align__(16) float sRow[64];         // the pivot row being broadcast
    const int i = threadIdx.x;
    {
        // 64 independent coalesced loads (row u, column i), then the stores
        float v[64];
#pragma unroll
        for (int u = 0; u < 64; ++u) v[u] = Pbuf[(o + u) * ld + o + i];
#pragma unroll
        for (int u = 0; u < 64; ++u) sT[u * 68 + i] = (i <= u) ? v[u] : 0.f;
    }
    __syncthreads();
    float s[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) s[j] = (j <= i) ? sT[i * 68 + j] : sT[j * 68 + i];

    int fail = -1;
    float my_rs = 0.f;
#pragma unroll
    for (int k = 63; k >= 0; --k) {
        if (i == k) {
#pragma unroll
            for (int q = 0; q <= k / 4; ++q) {
                f32x4 v;
                v.x = s[4 * q + 0];
                v.y = s[4 * q + 1];
                v.z = s[4 * q + 2];
                v.w = s[4 * q + 3];
                *reinterpret_cast<f32x4*>(sRow + 4 * q) = v;
            }
        }
        __syncthreads();
        const float piv = sRow[k];
        if (!(piv > 0.f) && fail < 0) fail = k;
        const float rs = __builtin_amdgcn_rsqf(piv);          // 1 / sqrt(piv)
        my_rs = (i == k) ? rs : my_rs;
        const float mul = (i < k) ? s[k] * (rs * rs) : 0.f;    // S[i][k] / S[k][k]
#pragma unroll
        for (int q = 0; 4 * q < k; ++q) {
            const f32x4 r = *reinterpret_cast<const f32x4*>(sRow + 4 * q);
            if (4 * q + 0 < k) s[4 * q + 0] = fmaf(-mul, r.x, s[4 * q + 0]);
            if (4 * q + 1 < k) s[4 * q + 1] = fmaf(-mul, r.y, s[4 * q + 1]);
            if (4 * q + 2 < k) s[4 * q + 2] = fmaf(-mul, r.z, s[4 * q + 2]);
            if (4 * q + 3 < k) s[4 * q + 3] = fmaf(-mul, r.w, s[4 * q + 3]);
        }
        __syncthreads();     // sRow is rewritten by the next step
    }
#pragma unroll
    for (int j = 0; j < 64; ++j) s[j] = (j <= i) ? s[j] * my_rs : 0.f;
    // lane i now holds row i of L (zeros above the diagonal); publish L^T
#pragma unroll
    for (int j = 0; j < 64; ++j) sT[j * 68 + i] = s[j];
    __syncthreads();
    float x[64];
#pragma unroll
    for (int j = 0; j < 64; ++j) x[j] = (j == i) ? __builtin_amdgcn_rcpf(s[j]) : 0.f;
#pragma unroll
    for (int j = 62; j >= 0; --j) {
        const f32x4* col = reinterpret_cast<const f32x4*>(sT + j * 68);
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int q = (j + 1) / 4; q < 16; ++q) {
            const f32x4 c = col[q];
            if (4 * q + 0 > j) a0 = fmaf(x[4 * q + 0], c.x, a0);
            if (4 * q + 1 > j) a1 = fmaf(x[4 * q + 1], c.y, a1);
            if (4 * q + 2 > j) a2 = fmaf(x[4 * q + 2], c.z, a2);
            if (4 * q + 3 > j) a3 = fmaf(x[4 * q + 3], c.w, a3);
        }
        const float v = -((a0 + a1) + (a2 + a3)) * __builtin_amdgcn_rcpf(sT[j * 68 + j]);
        x[j] = (j < i) ? v : x[j];
    }
    // coalesced stores of L (from L^T in LDS) and of X (via LDS)
    for (int idx = i; idx < 64 * 64; idx += 64) {
        const int r = idx >> 6, c = idx & 63;
        Lbuf[(o + r) * ld + o + c] = sT[c * 68 + r];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 64; ++j) sT[i * 68 + j] = x[j];
    __syncthreads();
    for (int idx = i; idx < 64 * 64; idx += 64) {
        const int r = idx >> 6, c = idx & 63;
        Pbuf[(o + r) * ld + o + c] = sT[r * 68 + c];
    }
    if (i == 0 && fail >= 0) atomicCAS(info, 0, (int32_t)(o + fail + 1));
}

// ------------------------------------------------------ recursive GEMMs

constexpr int FBM = 128, FBN = 128;   // 128 x 128 output blocks

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

// A11 -= L21^T L21 on lower-triangular 128-blocks of the n1 x n1 block;
// only entries on or below the diagonal are written, so the strictly upper
// part of Pbuf stays zero (later products read whole triangular blocks).
__global__ __launch_bounds__(256) void k_f_syrk(const float* __restrict__ Lbuf, float* __restrict__ Pbuf,
                                                int64_t ld, int64_t o1, int64_t o2, int n1, int n2)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, KRow, KRow>::LDS_FLOATS];
    // linear block index -> (br, bc) with br >= bc
    const int q = blockIdx.x;
    int br = (int)((sqrtf(8.f * q + 1.f) - 1.f) * 0.5f);
    while ((br + 1) * (br + 2) / 2 <= q) ++br;
    while (br * (br + 1) / 2 > q) --br;
    const int bc = q - br * (br + 1) / 2;
    const int r0 = br * FBM, c0 = bc * FBN;
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, KRow, KRow>(Lbuf + o2 * ld + o1 + r0, ld, n1 - r0,
                                 Lbuf + o2 * ld + o1 + c0, ld, n1 - c0, 0, n2, lds, acc);
    block_store<2, 2>(Pbuf + (o1 + r0) * ld + o1 + c0, ld, n1 - r0, n1 - c0, -1.f, 1.f, acc, c0 - r0);
}

// T = L21 Li11 : (n2 x n1); Li11 is lower, so output columns from c0 need
// K in [c0, n1).
__global__ __launch_bounds__(256) void k_f_right(const float* __restrict__ Lbuf, const float* __restrict__ Pbuf,
                                                 float* __restrict__ T, int64_t ld, int64_t o1, int64_t o2,
                                                 int n1, int n2)
{
    __shared__ __align__(16) float lds[Gemm<2, 2, RowK, KRow>::LDS_FLOATS];
    const int r0 = blockIdx.y * FBM, c0 = blockIdx.x * FBN;
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

// P = Li diag(L) on and below the diagonal, zeros above, for L and P; when
// the factor ran in padded workspace, also copy the leading n x n out.
__global__ __launch_bounds__(256) void k_f_finish(float* __restrict__ Lbuf, float* __restrict__ Pbuf, int64_t ld,
                                                  int64_t Np, int64_t n, float* __restrict__ Lout,
                                                  float* __restrict__ Pout)
{
    for (int64_t i = blockIdx.y; i < Np; i += gridDim.y)
        for (int64_t j = blockIdx.x * 256 + threadIdx.x; j < Np; j += (int64_t)gridDim.x * 256) {
            float l = 0.f, p = 0.f;
            if (j <= i) {
                l = Lbuf[i * ld + j];
                p = Pbuf[i * ld + j] * Lbuf[j * ld + j];
            }
            if (Lout) {
                if (i < n && j < n) {
                    Lout[i * n + j] = l;
                    Pout[i * n + j] = p;
                }
            } else {
                Lbuf[i * ld + j] = l;
                Pbuf[i * ld + j] = p;
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
    if (nsz == kTile) {
        launch(R.prof, KK_F_BASE, 2.0 * 2.0 * 64.0 * 64.0 * 64.0 / 6.0, 4.0 * (tri(64) + 2 * 64 * 64),
               k_base_block, dim3(1), dim3(64), R.s, R.Lbuf, R.Pbuf, R.ld, o, R.info);
        return launch_ok();
    }
    const int64_t nt = nsz / kTile;
    const int n1 = (int)(kTile * (nt / 2));
    const int n2 = (int)(nsz - n1);
    const int64_t o1 = o, o2 = o + n1;
    const double d1 = n1, d2 = n2;
    if (factor_rec(R, o2, n2)) return -1;
    {
        dim3 g((unsigned)ceil_div(n1, FBN), (unsigned)ceil_div(n2, FBM));
        launch(R.prof, KK_F_PANEL, 2.0 * d1 * tri(d2), 4.0 * (tri(d2) + 2.0 * d2 * d1), k_f_panel, g, dim3(256),
               R.s, R.Pbuf, R.Lbuf, R.ld, o1, o2, n1, n2);
    }
    {
        const int64_t tb = ceil_div(n1, FBM);
        launch(R.prof, KK_F_SYRK, 2.0 * d2 * tri(d1), 4.0 * (d2 * d1 + 2.0 * tri(d1)), k_f_syrk,
               dim3((unsigned)(tb * (tb + 1) / 2)), dim3(256), R.s, R.Lbuf, R.Pbuf, R.ld, o1, o2, n1, n2);
    }
    if (launch_ok()) return -1;
    if (factor_rec(R, o1, n1)) return -1;
    {
        dim3 g((unsigned)ceil_div(n1, FBN), (unsigned)ceil_div(n2, FBM));
        launch(R.prof, KK_F_RIGHT, 2.0 * d2 * tri(d1), 4.0 * (2.0 * d2 * d1 + tri(d1)), k_f_right, g, dim3(256),
               R.s, R.Lbuf, R.Pbuf, R.T, R.ld, o1, o2, n1, n2);
        launch(R.prof, KK_F_LEFT, 2.0 * d1 * tri(d2), 4.0 * (2.0 * d2 * d1 + tri(d2)), k_f_left, g, dim3(256),
               R.s, R.T, R.Pbuf, R.ld, o1, o2, n1, n2);
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

    launch(prof, KK_F_PREP, 0.0, 4.0, k_clear_info, dim3(1), dim3(64), s, info);
    launch(prof, KK_F_PREP, 0.0, 4.0 * dn, k_diag_mean, dim3(1), dim3(256), s, A, n, mean);
    {
        dim3 g((unsigned)ceil_div(p.Np, 256), (unsigned)std::min<int64_t>(p.Np, 32768));
        launch(prof, KK_F_PREP, dn, 4.0 * (tri(dn) + dN * dN), k_load_damped, g, dim3(256), s, A, n, R.Pbuf,
               p.Np, p.Np, (const float*)mean, damp_frac);
    }
    if (launch_ok()) return -1;
    if (factor_rec(R, 0, p.Np)) return -1;
    {
        dim3 g((unsigned)ceil_div(p.Np, 256), (unsigned)std::min<int64_t>(p.Np, 32768));
        launch(prof, KK_F_FINISH, dn * dn / 2.0, 4.0 * (2.0 * tri(dN) + 2.0 * dn * dn), k_f_finish, g, dim3(256),
               s, R.Lbuf, R.Pbuf, p.Np, p.Np, n, p.padded ? L : (float*)nullptr, p.padded ? P : (float*)nullptr);
    }
    return launch_ok();
}

}  // namespace bk
