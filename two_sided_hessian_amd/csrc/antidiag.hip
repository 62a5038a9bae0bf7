// antidiag.hip -- BaKron-antidiagonal on gfx950: the rounding of W (m x n)
// under A (x) B, one entry anti-diagonal at a time.
//
// Method (paper summary "FastKron: Efficient Quantization with
// Kronecker-Factored Hessians", derivation, second variant, and Theorem 3.2;
// Table 3 times it against BaKron): entries (i, j) with i + j = k do not
// update one another, so the whole anti-diagonal D_k is rounded at once and
// its raw errors E_k are pushed into the rest of the matrix with one
// rank-|D_k| product,
//     W~ -= P_B E_k P_A^T,
// which only reaches entries below and to the right of a source (P_A, P_B
// lower triangular).  m + n - 1 dependent steps and about m^2 n^2 / 2
// multiply-adds in all (every entry pushes into its whole bottom-right
// block), against mn(m + n) / 2 for the divide and conquer of bakron_solve;
// the result is the same rounding (Theorem 3.2).
//
// Per step k (sources i in [i0, i1], j = k - i):
//  * k_ad_quant, one workgroup per row r of the step's K range: the row's
//    entry on D_k is rounded exactly as the solve's leaf rounds (correctly
//    rounded w / s by Markstein's correction, x = q + z, round half to even,
//    clamp), and the row's stage-1 product is written:
//        Y[r, c] = e_r P_A[c, k - r]   (r on D_k),   0 (other rows),
//    read from a transposed copy of P_A so that the row is contiguous;
//  * k_ad_update, one 128 x 128 target block per workgroup, fp32 MFMA:
//        W~[block] -= P_B[block rows, K] Y[K, block cols],
//    with K the sources that can reach the block: i <= the block's last row
//    (P_B lower triangular) and k - i <= its last column (P_A lower
//    triangular), rounded out to 32-row chunks (the rows added by the
//    rounding hold zeros in Y).  Blocks with no entry past the anti-diagonal
//    return at once.
// Extra products with exact zeros (P_B above its diagonal, Y outside D_k)
// add nothing, so entries already rounded keep their values.
//
// Workspace (Mp = 64 ceil(m / 64), Np = 64 ceil(n / 64)):
//   Wt  Mp x Np  working weights (W copied in, zero padded)
//   Y   Mp x Np  the step's stage-1 rows
//   PAT Np x Np  P_A transposed (zero padded)
//   PBp Mp x Mp  padded copy of P_B (only when m is not a multiple of 64)
//   obj Mp doubles: per-row objective sums
#include <algorithm>

#include "gemm.hpp"
#include "internal.hpp"

namespace bk {

namespace {

constexpr int kAdBlock = 128;   // target block edge of k_ad_update

// dst (R x C, pitch ldd) = src (rows x cols, pitch lds), zeros outside.
__global__ __launch_bounds__(256) void k_ad_copy(const float* __restrict__ src, int64_t rows, int64_t cols,
                                                 int64_t lds, float* __restrict__ dst, int64_t R, int64_t C,
                                                 int64_t ldd)
{
    for (int64_t i = blockIdx.y; i < R; i += gridDim.y)
        for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < C; j += (int64_t)gridDim.x * 256)
            dst[i * ldd + j] = (i < rows && j < cols) ? src[i * lds + j] : 0.f;
}

// PAT[j][c] = P_A[c][j] for j, c < n, zero elsewhere in Np x Np; 32 x 32
// tiles through LDS so that reads and writes are both row-contiguous.
__global__ __launch_bounds__(256) void k_ad_transpose(const float* __restrict__ PA, int64_t n,
                                                      float* __restrict__ PAT, int64_t Np)
{
    __shared__ float t[32][33];
    const int64_t c0 = (int64_t)blockIdx.x * 32, j0 = (int64_t)blockIdx.y * 32;   // source rows c, columns j
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;                     // 32 x 8 threads
    for (int r = ty; r < 32; r += 8) {
        const int64_t c = c0 + r, j = j0 + tx;
        t[r][tx] = (c < n && j < n) ? PA[c * n + j] : 0.f;
    }
    __syncthreads();
    for (int r = ty; r < 32; r += 8) PAT[(j0 + r) * Np + c0 + tx] = t[tx][r];
}

__global__ __launch_bounds__(256) void k_ad_fill(double* __restrict__ p, int64_t count)
{
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) p[i] = 0.0;
}

struct AdArgs {
    float* Wt;            // Mp x Np (pitch Np)
    float* Y;             // Mp x Np (pitch Np)
    const float* PAT;     // Np x Np
    int64_t Np;
    const float* scale;
    const float* zero;
    const int32_t* maxq;
    int m, n;
    uint8_t* codes;       // m x n outputs (pitch n)
    float* V;
    float* err;           // nullable
    const float* LA;      // nullable with obj
    const float* LB;
    double* obj;          // nullable: per-row objective sums
};

// Step k: workgroup b handles row r = R0 + b; rounds (r, k - r) when r is on
// the anti-diagonal and writes Y[r, c0 .. Np).
__global__ __launch_bounds__(256) void k_ad_quant(AdArgs g, int k, int i0, int i1, int R0, int64_t c0)
{
    __shared__ float se;
    const int r = R0 + (int)blockIdx.x;
    const bool src = r >= i0 && r <= i1;
    if (threadIdx.x == 0) {
        float e = 0.f;
        if (src) {
            const int j = k - r;
            const float w = g.Wt[(int64_t)r * g.Np + j];
            const float sc = g.scale[r], zc = g.zero[r], mq = (float)g.maxq[r];
            const float sinv = 1.f / sc;   // correctly rounded
            // w / sc correctly rounded (Markstein), then x = RN(q + zc)
            float q0 = w * sinv;
            const float rem = fmaf(-q0, sc, w);
            q0 = fmaf(rem, sinv, q0);
            const float x = q0 + zc;
            const float c = fminf(fmaxf(rintf(x), 0.f), mq);
            const float v = sc * (c - zc);
            e = w - v;
            const int64_t o = (int64_t)r * g.n + j;
            g.codes[o] = (uint8_t)c;
            g.V[o] = v;
            if (g.err) g.err[o] = e;
            if (g.obj) {
                const double q = (double)g.LB[(int64_t)r * g.m + r] * (double)g.LA[(int64_t)j * g.n + j] * (double)e;
                g.obj[r] += q * q;
            }
        }
        se = e;
    }
    __syncthreads();
    const float e = se;
    float* yr = g.Y + (int64_t)r * g.Np;
    if (src) {
        const float* pr = g.PAT + (int64_t)(k - r) * g.Np;   // P_A[c][k - r] for every c
        for (int64_t c = c0 + 4 * threadIdx.x; c < g.Np; c += 1024) {
            const f32x4 p = *reinterpret_cast<const f32x4*>(pr + c);
            *reinterpret_cast<f32x4*>(yr + c) = f32x4{e * p.x, e * p.y, e * p.z, e * p.w};
        }
    } else {
        for (int64_t c = c0 + 4 * threadIdx.x; c < g.Np; c += 1024)
            *reinterpret_cast<f32x4*>(yr + c) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// K rows (sources) that reach target block (rows r0 .., cols c0 ..) at step
// k, rounded out to kBK chunks: [kb, ke); false when there are none or every
// entry of the block is on or before the anti-diagonal.
__device__ __forceinline__ bool ad_krange(int k, int i0, int i1, int64_t r0, int64_t c0, int& kb, int& ke)
{
    const int64_t rlast = r0 + kAdBlock - 1, clast = c0 + kAdBlock - 1;
    if (rlast + clast <= k) return false;
    const int64_t lo = std::max<int64_t>(i0, (int64_t)k - clast);
    const int64_t hi = std::min<int64_t>(i1, rlast);
    if (lo > hi) return false;
    kb = (int)(lo / kBK * kBK);
    ke = (int)((hi / kBK + 1) * kBK);
    return true;
}

typedef Gemm<2, 2, RowK, KRow> AdBlk;

// Step k: blocks (bx, by) of the target grid starting at block column J0,
// block row I0; W~[block] -= P_B[block rows, K] Y[K, block cols].
__global__ __launch_bounds__(256, 2) void k_ad_update(float* __restrict__ Wt, const float* __restrict__ Y,
                                                      const float* __restrict__ PB, int64_t ldb, int64_t Mp,
                                                      int64_t Np, int k, int i0, int i1, int I0, int J0)
{
    __shared__ __align__(16) float lds[AdBlk::LDS_FLOATS];
    const int64_t r0 = (int64_t)(I0 + (int)blockIdx.y) * kAdBlock;
    const int64_t c0 = (int64_t)(J0 + (int)blockIdx.x) * kAdBlock;
    int kb, ke;
    if (!ad_krange(k, i0, i1, r0, c0, kb, ke)) return;
    const int rlim = (int)std::min<int64_t>(kAdBlock, Mp - r0), clim = (int)std::min<int64_t>(kAdBlock, Np - c0);
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, RowK, KRow>(PB + r0 * ldb, ldb, rlim, Y + c0, Np, clim, kb, ke, lds, acc);
    block_store<2, 2>(Wt + r0 * Np + c0, Np, rlim, clim, -1.f, 1.f, acc);
}

__global__ __launch_bounds__(256) void k_ad_obj(const double* __restrict__ part, int64_t count,
                                                double* __restrict__ out)
{
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < count; i += 256) s += part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[0] = red[0];
}

struct AdPlan {
    int64_t Mp, Np;
    bool pad_b;
    size_t off_wt, off_y, off_pat, off_pb, off_obj, total;
};

AdPlan plan_ad(int64_t m, int64_t n)
{
    AdPlan p;
    p.Mp = ceil_div(m, kTile) * kTile;
    p.Np = ceil_div(n, kTile) * kTile;
    p.pad_b = (m % kTile) != 0;
    const size_t mat = sizeof(float) * (size_t)(p.Mp * p.Np);
    size_t off = 0;
    p.off_wt = off;
    off = align_up(off + mat);
    p.off_y = off;
    off = align_up(off + mat);
    p.off_pat = off;
    off = align_up(off + sizeof(float) * (size_t)(p.Np * p.Np));
    p.off_pb = 0;
    if (p.pad_b) {
        p.off_pb = off;
        off = align_up(off + sizeof(float) * (size_t)(p.Mp * p.Mp));
    }
    p.off_obj = off;
    off = align_up(off + sizeof(double) * (size_t)p.Mp);
    p.total = off;
    return p;
}

dim3 grid2(int64_t R, int64_t C) { return dim3((unsigned)std::min<int64_t>(ceil_div(C, 256), 64), (unsigned)std::min<int64_t>(R, 32768)); }

}  // namespace

size_t antidiag_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0) return 0;
    return plan_ad(m, n).total;
}

int antidiag_enqueue(const float* W, int64_t m, int64_t n, const float* LA, const float* PA, const float* LB,
                     const float* PB, const float* scale, const float* zero, const int32_t* maxq, float* V,
                     uint8_t* codes, float* err, double* objective, void* ws, hipStream_t s, Prof* prof)
{
    const AdPlan p = plan_ad(m, n);
    char* w = static_cast<char*>(ws);
    AdArgs g;
    g.Wt = reinterpret_cast<float*>(w + p.off_wt);
    g.Y = reinterpret_cast<float*>(w + p.off_y);
    float* pat = reinterpret_cast<float*>(w + p.off_pat);
    g.PAT = pat;
    g.Np = p.Np;
    g.scale = scale;
    g.zero = zero;
    g.maxq = maxq;
    g.m = (int)m;
    g.n = (int)n;
    g.codes = codes;
    g.V = V;
    g.err = err;
    g.LA = LA;
    g.LB = LB;
    g.obj = objective ? reinterpret_cast<double*>(w + p.off_obj) : nullptr;
    const double dm = (double)m, dn = (double)n;
    launch(prof, KK_AD_PREP, 0.0, 4.0 * (dm * dn + (double)(p.Mp * p.Np)), k_ad_copy, grid2(p.Mp, p.Np), dim3(256),
           s, W, m, n, n, g.Wt, p.Mp, p.Np, p.Np);
    launch(prof, KK_AD_PREP, 0.0, 4.0 * (dn * dn + (double)(p.Np * p.Np)), k_ad_transpose,
           dim3((unsigned)(p.Np / 32), (unsigned)(p.Np / 32)), dim3(256), s, PA, n, pat, p.Np);
    const float* pb = PB;
    int64_t ldb = m;
    if (p.pad_b) {
        float* pbp = reinterpret_cast<float*>(w + p.off_pb);
        launch(prof, KK_AD_PREP, 0.0, 4.0 * (dm * dm + (double)(p.Mp * p.Mp)), k_ad_copy, grid2(p.Mp, p.Mp),
               dim3(256), s, PB, m, m, m, pbp, p.Mp, p.Mp, p.Mp);
        pb = pbp;
        ldb = p.Mp;
    }
    if (g.obj)
        launch(prof, KK_AD_PREP, 0.0, 8.0 * (double)p.Mp, k_ad_fill, dim3((unsigned)ceil_div(p.Mp, 256)), dim3(256),
               s, g.obj, p.Mp);
    if (hipGetLastError() != hipSuccess) return -1;
    const int64_t Mb = ceil_div(p.Mp, kAdBlock), Nb = ceil_div(p.Np, kAdBlock);
    for (int k = 0; k <= (int)(m + n - 2); ++k) {
        const int i0 = (int)std::max<int64_t>(0, k - n + 1), i1 = (int)std::min<int64_t>(m - 1, k);
        const int R0 = i0 / kBK * kBK;
        const int R1 = (int)std::min<int64_t>(p.Mp, (int64_t)(i1 / kBK + 1) * kBK);
        // targets: block rows from the first source's, block columns from
        // the first column a source reaches (k - i1)
        const int I0 = i0 / kAdBlock, J0 = (k - i1) / kAdBlock;
        const int64_t c0 = (int64_t)J0 * kAdBlock;
        double qfl = 0.0;
        if (prof) qfl = 2.0 * (double)(i1 - i0 + 1);
        launch(prof, KK_AD_QUANT, qfl, 4.0 * (double)(R1 - R0) * (double)(p.Np - c0) * 2.0, k_ad_quant,
               dim3((unsigned)(R1 - R0)), dim3(256), s, g, k, i0, i1, R0, c0);
        double fl = 0.0, by = 0.0;
        if (prof) {
            // the block products the launch executes (K rounded out to chunks)
            for (int64_t bi = I0; bi < Mb; ++bi)
                for (int64_t bj = J0; bj < Nb; ++bj) {
                    const int64_t r0 = bi * kAdBlock, cc = bj * kAdBlock;
                    if (r0 + cc + 2 * kAdBlock - 2 <= k) continue;
                    const int64_t lo = std::max<int64_t>(i0, k - (cc + kAdBlock - 1));
                    const int64_t hi = std::min<int64_t>(i1, r0 + kAdBlock - 1);
                    if (lo > hi) continue;
                    const double kl = (double)((hi / kBK + 1) * kBK - lo / kBK * kBK);
                    fl += 2.0 * kAdBlock * kAdBlock * kl;
                    by += 4.0 * (2.0 * kAdBlock * kl + 2.0 * kAdBlock * kAdBlock);
                }
        }
        launch(prof, KK_AD_UPDATE, fl, by, k_ad_update, dim3((unsigned)(Nb - J0), (unsigned)(Mb - I0)), dim3(256),
               s, g.Wt, (const float*)g.Y, pb, ldb, p.Mp, p.Np, k, i0, i1, I0, J0);
        if ((k & 255) == 0 && hipGetLastError() != hipSuccess) return -1;
    }
    if (hipGetLastError() != hipSuccess) return -1;
    if (objective) {
        launch(prof, KK_AD_PREP, dm, 8.0 * (dm + 1.0), k_ad_obj, dim3(1), dim3(256), s, (const double*)g.obj,
               (int64_t)m, objective);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

}  // namespace bk
