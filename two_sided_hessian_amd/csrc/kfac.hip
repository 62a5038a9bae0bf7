// kfac.hip -- Kronecker factors of the layer Hessian from per-sample inputs, for gfx950.
//
// Method (paper summary "FastKron: Efficient Quantization with
// Kronecker-Factored Hessians", Hessian choices): with per-sample input
// activations a_t (n) and output gradients b_t (m), the Hessian of the layer
// is approximated by A (x) B in one of two ways:
//   * K-FAC-style independence:  A = E[a a^T],         B = E[b b^T];
//   * Shampoo-style, one power-iteration step of the nearest Kronecker
//     product from the identity:  A = E[|b|^2 a a^T],  B = E[|a|^2 b b^T].
// Both are weighted second moments  M = scale * sum_t w_t x_t x_t^T  of a
// sample-major matrix X (row t = x_t), with w_t = 1 or w_t = |y_t|^2 from the
// other side's samples, and scale = 1 / N.
//
// MI355X layout:
//  * k_row_sqnorms: one wave per sample row, float4 loads, wave reduction.
//    Streams X once (HBM bound).
//  * k_moment: the lower block triangle of M in 128 x 128 output blocks
//    (fp32 MFMA, v_mfma_f32_32x32x2f32, four waves of 64 x 64), K running
//    over the samples in chunks of 32 staged through LDS.  Both operands are
//    column strips of X, feature-contiguous in memory, so the LDS copy is a
//    straight float4 move; the chunk's 32 weights w_t are staged beside them
//    and scale one operand's MFMA fragments as they are read (four weights
//    per 16-byte LDS read).  Only the lower triangle and the diagonal of M
//    are written: the factor step reads nothing else.
#include <algorithm>
#include <math.h>

#include "gemm.hpp"
#include "internal.hpp"

namespace bk {

// out[t] = sum_i X[t, i]^2; 256 threads = 4 rows per workgroup.
__global__ __launch_bounds__(256) void k_row_sqnorms(const float* __restrict__ X, int64_t N, int64_t n,
                                                     float* __restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= N) return;
    const float* row = X + t * n;
    float s = 0.f;
    for (int64_t i = 4 * lane; i < n; i += 256) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(row + i);
        s = fmaf(v.x, v.x, s);
        s = fmaf(v.y, v.y, s);
        s = fmaf(v.z, v.z, s);
        s = fmaf(v.w, v.w, s);
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) out[t] = s;
}

constexpr int kMB = 128;                      // output block edge
typedef Operand<kMB, KRow> MomOp;             // LDS [k][r], pitch 128 + 4

// One K chunk of a column strip of X into registers: float4 u of this thread
// holds X[k0 + k, c0 + r .. r + 3] (zero beyond N or n).  n is a multiple of
// 4, so a float4 never straddles n.
__device__ __forceinline__ void mom_load(const float* __restrict__ X, int64_t N, int64_t n, int64_t c0, int64_t k0,
                                         f32x4 (&reg)[MomOp::PER_THREAD])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < MomOp::PER_THREAD; ++u) {
        const int f = t + 256 * u;
        const int k = f / (kMB / 4), r = 4 * (f % (kMB / 4));
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (k0 + k < N && c0 + r < n) v = *reinterpret_cast<const f32x4*>(X + (k0 + k) * n + c0 + r);
        reg[u] = v;
    }
}

// Lower block (bi, bj), bi >= bj, from the block index p = bi (bi + 1) / 2 + bj.
__device__ __forceinline__ void lower_block(unsigned p, int& bi, int& bj)
{
    int i = (int)((sqrtf(8.f * (float)p + 1.f) - 1.f) * 0.5f);
    while ((unsigned)(i * (i + 1) / 2) > p) --i;
    while ((unsigned)((i + 1) * (i + 2) / 2) <= p) ++i;
    bi = i;
    bj = (int)p - i * (i + 1) / 2;
}

// Workgroups are dealt to the eight XCDs round-robin; consecutive blocks of
// one block row share the weighted operand strip, so each run of 32
// workgroups is permuted to give every XCD four consecutive blocks.
__device__ __forceinline__ unsigned xcd_run4(unsigned p, unsigned n)
{
    if (p >= n / 32u * 32u) return p;
    const unsigned r = p % 32u;
    return p - r + (r % 8u) * 4u + r / 8u;
}

template <bool W>
__global__ __launch_bounds__(256) void k_moment(const float* __restrict__ X, int64_t N, int64_t n,
                                                const float* __restrict__ w, float scale, float* __restrict__ M)
{
    __shared__ __align__(16) float lds[2 * MomOp::FLOATS];
    __shared__ __align__(16) float sw[kBK];   // weights of the staged chunk
    int bi, bj;
    lower_block(xcd_run4(blockIdx.x, gridDim.x), bi, bj);
    const int64_t r0 = (int64_t)bi * kMB, c0 = (int64_t)bj * kMB;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wy = wave >> 1, wx = wave & 1;
    const int ml = lane & 31;
    float* sa = lds;
    float* sb = lds + MomOp::FLOATS;

    Acc acc;
    acc_zero(acc);
    f32x4 ra[MomOp::PER_THREAD], rb[MomOp::PER_THREAD];
    const int t = threadIdx.x;
    float wr = 0.f;   // thread t < kBK: weight of sample k0 + t of the chunk in flight
    const int64_t nchunk = (N + kBK - 1) / kBK;
    mom_load(X, N, n, r0, 0, ra);
    mom_load(X, N, n, c0, 0, rb);
    if (W && t < kBK) wr = t < N ? w[t] : 0.f;
    MomOp::store(sa, ra);
    MomOp::store(sb, rb);
    if (W && t < kBK) sw[t] = wr;
    __syncthreads();
    for (int64_t c = 0; c < nchunk; ++c) {
        const bool more = (c + 1) < nchunk;
        if (more) {
            const int64_t k1 = (c + 1) * kBK;
            mom_load(X, N, n, r0, k1, ra);
            mom_load(X, N, n, c0, k1, rb);
            if (W && t < kBK) wr = k1 + t < N ? w[k1 + t] : 0.f;
        }
#pragma unroll
        for (int kc = 0; kc < kBK; kc += 8) {
            f32x4 a0 = MomOp::frag(sa, wy * 64 + ml, kc);
            f32x4 a1 = MomOp::frag(sa, wy * 64 + 32 + ml, kc);
            if (W) {   // element q of a fragment is sample kc + 4 (lane / 32) + q
                const f32x4 wq = *reinterpret_cast<const f32x4*>(sw + kc + 4 * (lane >> 5));
                a0 *= wq;
                a1 *= wq;
            }
            const f32x4 b0 = MomOp::frag(sb, wx * 64 + ml, kc);
            const f32x4 b1 = MomOp::frag(sb, wx * 64 + 32 + ml, kc);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[q], b0[q], acc.c[0][0], 0, 0, 0);
                acc.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[q], b1[q], acc.c[0][1], 0, 0, 0);
                acc.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[q], b0[q], acc.c[1][0], 0, 0, 0);
                acc.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[q], b1[q], acc.c[1][1], 0, 0, 0);
            }
        }
        if (more) {
            __syncthreads();
            MomOp::store(sa, ra);
            MomOp::store(sb, rb);
            if (W && t < kBK) sw[t] = wr;
            __syncthreads();
        }
    }
    // lower triangle and diagonal only, inside n
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = r0 + wy * 64 + acc_row(mi, r);
                const int64_t col = c0 + wx * 64 + acc_col(ni);
                if (row < n && col <= row) M[row * n + col] = scale * acc.c[mi][ni][r];
            }
}

// ------------------------------------------------------------ host side

int sqnorms_enqueue(const float* X, int64_t N, int64_t n, float* out, hipStream_t s, Prof* prof)
{
    launch(prof, KK_K_SQNORM, 2.0 * (double)N * (double)n, 4.0 * (double)N * ((double)n + 1.0), k_row_sqnorms,
           dim3((unsigned)ceil_div(N, 4)), dim3(256), s, X, N, n, out);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int moment_enqueue(const float* X, int64_t N, int64_t n, const float* w, float scale, float* M, hipStream_t s,
                   Prof* prof)
{
    const int64_t nb = ceil_div(n, kMB);
    const int64_t blocks = nb * (nb + 1) / 2;
    // algorithmic: the lower triangle and diagonal, n (n + 1) / 2 dot
    // products of length N (plus the weights); X read once, M written once
    const double fl = 2.0 * (double)N * (double)n * ((double)n + 1.0) / 2.0 + (w ? (double)N * (double)n : 0.0);
    const double by = 4.0 * ((double)N * (double)n + (double)n * ((double)n + 1.0) / 2.0 + (w ? (double)N : 0.0));
    if (w)
        launch(prof, KK_K_MOMENT_W, fl, by, k_moment<true>, dim3((unsigned)blocks), dim3(256), s, X, N, n, w, scale, M);
    else
        launch(prof, KK_K_MOMENT, fl, by, k_moment<false>, dim3((unsigned)blocks), dim3(256), s, X, N, n, w, scale, M);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace bk
