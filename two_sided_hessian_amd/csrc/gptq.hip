// gptq.hip -- the one-sided case B = I (GPTQ) of the BaKron rounding, for gfx950.
//
// Method (paper summary "FastKron: Efficient Quantization with
// Kronecker-Factored Hessians": setup, where GPTQ is the Hessian A (x) I, and
// the BaKron-naive update): quantizing entry (i, j) with raw error e changes
// entry (i', j') by -e P_B[i', i] P_A[j', j].  With B = I, P_B = I, so the
// update stays inside row i: rows are independent and only the column order
// matters.  Column j of every row is rounded at step j, then e P_A[j', j] is
// subtracted from every later column j' of the same row.  That is n dependent
// steps with all m rows in parallel (against m + n - 1 anti-diagonals of
// 64 x 64 tiles for a general B), and O(m n^2) work.
//
// MI355X layout:
//  * 64-column blocks; the block range is halved recursively: solve the left
//    half, subtract E[:, left] P_A[right, left]^T from the right half (one
//    dense fp32 MFMA GEMM, no staircase: P_A[right, left] is a full block of
//    the lower triangle), solve the right half.
//  * A leaf sweeps one 64-column block for 32 rows per workgroup: 8 lanes per
//    row, 8 columns per lane held in registers, the block's diagonal P_A
//    block in LDS.  The 64 steps are unrolled, so the lane and register that
//    hold column j are compile-time constants: the value is broadcast to the
//    row's 8 lanes with two DPP moves, rounded by every lane, and each lane
//    subtracts e P_A[c, j] from its 8 columns c (P_A is zero above its
//    diagonal, so earlier columns are left alone without a test).  Rows never
//    exchange data, so a step needs no barrier.
//
// Workspace (Mp = 64 ceil(m / 64), Np = 64 ceil(n / 64)):
//   Wt  Mp x Np  working weights (W copied in, zero padded)
//   E   Mp x Np  raw errors
//   obj Nt x (Mp / 32) per-(column block, workgroup) objective partials
//   PAp Np x Np  padded copy of P_A, only when n is not a multiple of 64
#include <algorithm>

#include <limits.h>

#include "gemm.hpp"
#include "internal.hpp"

namespace bk {

constexpr int kGRows = 32;   // rows per sweep workgroup
constexpr int kGP = 68;      // LDS pitch (floats) of the transposed P_A block

// dst (R x C, pitch ldd) = src (rows x cols, pitch lds) with zeros outside.
// C and ldd are multiples of 4: four adjacent columns per thread, one
// 16-byte store, and one 16-byte load where they lie inside src and src's
// rows are 16-byte aligned (vec).
__global__ __launch_bounds__(256) void k_gptq_load(const float* __restrict__ src, int64_t rows, int64_t cols,
                                                   int64_t lds, float* __restrict__ dst, int64_t R, int64_t C,
                                                   int64_t ldd, int vec)
{
    for (int64_t i = blockIdx.y; i < R; i += gridDim.y)
        for (int64_t j = 4 * ((int64_t)blockIdx.x * 256 + threadIdx.x); j < C; j += (int64_t)gridDim.x * 1024) {
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (i < rows) {
                if (vec && j + 3 < cols) {
                    v = *reinterpret_cast<const f32x4*>(src + i * lds + j);
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (j + q < cols) v[q] = src[i * lds + j + q];
                }
            }
            *reinterpret_cast<f32x4*>(dst + i * ldd + j) = v;
        }
}

struct SweepArgs {
    float* Wt;            // Mp x Np working weights (pitch ldw)
    float* E;             // Mp x Np raw errors (pitch ldw)
    int64_t ldw;
    const float* PA;      // P_A (pitch lda)
    int64_t lda;
    const float* scale;   // grid of row i in this column block: index i * gld + gcol
    const float* zero;
    const int32_t* maxq;
    int64_t gld;          // grid pitch: 1 (per row) or the number of column groups
    int gtiles;           // 64-column blocks per column group (huge for per-row grids)
    int m, n;
    uint8_t* codes;       // m x n outputs (pitch n)
    float* V;
    float* err;           // nullable
    const float* LA;      // nullable: diagonal source for the objective (pitch n)
    double* objp;         // nullable: partials of this column block, one per workgroup
    int J;                // column block
    int vec_out;          // outputs may use 16-byte / 8-byte stores
};

// Value of register x in lane O (0..7) of this lane's group of 8, in every
// lane of the group.  Quad broadcast first, then the other quad of the group
// takes it over with a 4-lane row shift (bank_mask picks the receiving quads).
template <int O>
__device__ __forceinline__ float bcast8(float x)
{
    constexpr int q = O & 3;
    constexpr int perm = q | (q << 2) | (q << 4) | (q << 6);
    const int xi = __builtin_bit_cast(int, x);
    const int b = __builtin_amdgcn_mov_dpp(xi, perm, 0xF, 0xF, false);
    // O < 4: quads 1 and 3 of each 16-lane row read lane - 4 (row_shr:4);
    // O >= 4: quads 0 and 2 read lane + 4 (row_shl:4).
    const int r = (O < 4) ? __builtin_amdgcn_update_dpp(b, b, 0x114, 0xF, 0xA, false)
                          : __builtin_amdgcn_update_dpp(b, b, 0x104, 0xF, 0x5, false);
    return __builtin_bit_cast(float, r);
}

// One step of the sweep: column j = 8 O + K of the block.  `pc` holds this
// step's P_A column (read one step earlier); the next step's column is read
// first, so its LDS latency overlaps this step's arithmetic.
template <int O, int K>
__device__ __forceinline__ void sweep_step(float (&w)[8], float (&ev)[8], float (&cv)[8], f32x4 (&pc)[2],
                                           const float* __restrict__ sPT, int sg, float sc, float sinv, float zc,
                                           float mq, int ncols)
{
    constexpr int j = 8 * O + K;
    f32x4 pn[2];
    if (j + 1 < 64) {
        pn[0] = *reinterpret_cast<const f32x4*>(sPT + (j + 1) * kGP + 8 * sg);
        pn[1] = *reinterpret_cast<const f32x4*>(sPT + (j + 1) * kGP + 8 * sg + 4);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float wj = bcast8<O>(w[K]);
    // wj / sc correctly rounded (Markstein: with y = RN(1/sc), q0 = RN(wj y)
    // is within an ulp, the remainder is exact under fma, RN(q0 + r y) is
    // RN(wj / sc)); then x = RN(q + zc), round half to even, clamp.
    float q0 = wj * sinv;
    const float rem = fmaf(-q0, sc, wj);
    q0 = fmaf(rem, sinv, q0);
    const float x = q0 + zc;
    const float c = fminf(fmaxf(rintf(x), 0.f), mq);
    const float v = sc * (c - zc);
    const float e = (j < ncols) ? (wj - v) : 0.f;
    // P_A[c, j] for this lane's columns c = 8 sg + k: zero for c < j, one at
    // c == j (the owner's own entry, never read again), the update for c > j.
    w[0] = fmaf(-e, pc[0].x, w[0]);
    w[1] = fmaf(-e, pc[0].y, w[1]);
    w[2] = fmaf(-e, pc[0].z, w[2]);
    w[3] = fmaf(-e, pc[0].w, w[3]);
    w[4] = fmaf(-e, pc[1].x, w[4]);
    w[5] = fmaf(-e, pc[1].y, w[5]);
    w[6] = fmaf(-e, pc[1].z, w[6]);
    w[7] = fmaf(-e, pc[1].w, w[7]);
    if (sg == O) {
        ev[K] = e;
        cv[K] = c;
    }
    if (j + 1 < 64) {
        pc[0] = pn[0];
        pc[1] = pn[1];
    }
}

template <int O>
__device__ __forceinline__ void sweep_group(float (&w)[8], float (&ev)[8], float (&cv)[8], f32x4 (&pc)[2],
                                            const float* __restrict__ sPT, int sg, float sc, float sinv, float zc,
                                            float mq, int ncols)
{
    sweep_step<O, 0>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 1>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 2>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 3>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 4>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 5>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 6>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_step<O, 7>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
}

// Column block J for rows 32 blockIdx.x .. + 31; 256 threads = 32 rows x 8 lanes.
__global__ __launch_bounds__(256) void k_gptq_sweep(SweepArgs g)
{
    __shared__ __align__(16) float sPT[64 * kGP];   // sPT[j][c] = P_A[c0 + c][c0 + j]
    __shared__ double sRed[4];
    const int t = threadIdx.x;
    const int row = t >> 3, sg = t & 7;
    const int64_t r0 = (int64_t)blockIdx.x * kGRows;
    const int64_t c0 = (int64_t)g.J * 64;

    // diagonal P_A block, transposed into LDS (rows of the block are read
    // as float4s and scattered down the columns of sPT)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int f = t + 256 * u;
        const int c = f >> 4, jq = 4 * (f & 15);
        const f32x4 p = *reinterpret_cast<const f32x4*>(g.PA + (c0 + c) * g.lda + c0 + jq);
        sPT[(jq + 0) * kGP + c] = p.x;
        sPT[(jq + 1) * kGP + c] = p.y;
        sPT[(jq + 2) * kGP + c] = p.z;
        sPT[(jq + 3) * kGP + c] = p.w;
    }
    const int64_t grow = r0 + row;
    const float* wp = g.Wt + grow * g.ldw + c0 + 8 * sg;
    const f32x4 wa = *reinterpret_cast<const f32x4*>(wp);
    const f32x4 wb = *reinterpret_cast<const f32x4*>(wp + 4);
    float w[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
    const bool row_ok = grow < g.m;
    const int64_t gi = grow * g.gld + g.J / g.gtiles;   // the block lies in one column group
    const float sc = row_ok ? g.scale[gi] : 1.f;
    const float zc = row_ok ? g.zero[gi] : 0.f;
    const float mq = row_ok ? (float)g.maxq[gi] : 0.f;
    const float sinv = 1.f / sc;   // correctly rounded
    // columns of this block that exist (all 64 unless n is ragged); a
    // padding row keeps zero errors through col_ok = false
    const int64_t left = (int64_t)g.n - c0;
    const int ncols = row_ok ? (left < 64 ? (int)left : 64) : 0;
    float ev[8], cv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ev[k] = cv[k] = 0.f;
    __syncthreads();

    f32x4 pc[2];
    pc[0] = *reinterpret_cast<const f32x4*>(sPT + 8 * sg);
    pc[1] = *reinterpret_cast<const f32x4*>(sPT + 8 * sg + 4);
    sweep_group<0>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<1>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<2>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<3>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<4>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<5>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<6>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);
    sweep_group<7>(w, ev, cv, pc, sPT, sg, sc, sinv, zc, mq, ncols);

    // Outputs: raw errors to the workspace (padding entries are zero), codes /
    // values / errors to the caller, the objective partial.
    float* ep = g.E + grow * g.ldw + c0 + 8 * sg;
    *reinterpret_cast<f32x4*>(ep) = f32x4{ev[0], ev[1], ev[2], ev[3]};
    *reinterpret_cast<f32x4*>(ep + 4) = f32x4{ev[4], ev[5], ev[6], ev[7]};
    double objs = 0.0;
    if (row_ok) {
        const int64_t col0 = c0 + 8 * sg;
        const int64_t o = grow * g.n + col0;
        if (g.vec_out) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lo |= (uint32_t)cv[k] << (8 * k);
                hi |= (uint32_t)cv[k + 4] << (8 * k);
            }
            *reinterpret_cast<uint2*>(g.codes + o) = uint2{lo, hi};
            f32x4 va, vb;
            va.x = sc * (cv[0] - zc);
            va.y = sc * (cv[1] - zc);
            va.z = sc * (cv[2] - zc);
            va.w = sc * (cv[3] - zc);
            vb.x = sc * (cv[4] - zc);
            vb.y = sc * (cv[5] - zc);
            vb.z = sc * (cv[6] - zc);
            vb.w = sc * (cv[7] - zc);
            *reinterpret_cast<f32x4*>(g.V + o) = va;
            *reinterpret_cast<f32x4*>(g.V + o + 4) = vb;
            if (g.err) {
                *reinterpret_cast<f32x4*>(g.err + o) = f32x4{ev[0], ev[1], ev[2], ev[3]};
                *reinterpret_cast<f32x4*>(g.err + o + 4) = f32x4{ev[4], ev[5], ev[6], ev[7]};
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (col0 + k < g.n) {
                    g.codes[o + k] = (uint8_t)cv[k];
                    g.V[o + k] = sc * (cv[k] - zc);
                    if (g.err) g.err[o + k] = ev[k];
                }
            }
        }
        if (g.objp) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int64_t col = col0 + k;
                if (col < g.n) {
                    const double q = (double)g.LA[col * g.n + col] * (double)ev[k];
                    objs += q * q;
                }
            }
        }
    }
    if (g.objp) {
        for (int off = 32; off > 0; off >>= 1) objs += __shfl_xor(objs, off);
        if ((t & 63) == 0) sRed[t >> 6] = objs;
        __syncthreads();
        if (t == 0) g.objp[blockIdx.x] = sRed[0] + sRed[1] + sRed[2] + sRed[3];
    }
}

// ------------------------------------------------------ right-half update
//
// Wt[:, T] -= E[:, S] P_A[T, S]^T for the source block range S = [s0, s1) and
// the target range T = [t0, t1) (in columns, multiples of 64).  Both
// operands are K-contiguous (rows of E and rows of P_A run along S).

typedef Gemm<2, 2, RowK, RowK> UpdBlk;   // 128 x 128 output per workgroup

// Workgroups are dealt to the eight XCDs round-robin, and neighbouring
// output blocks along T share their E row strip: each run of 32 workgroups
// is permuted so that every XCD takes four consecutive blocks.
__device__ __forceinline__ unsigned xcd_group4(unsigned p, unsigned n)
{
    if (p >= n / 32u * 32u) return p;
    const unsigned r = p % 32u;
    return p - r + (r % 8u) * 4u + r / 8u;
}

__global__ __launch_bounds__(256, 2) void k_gptq_update(const float* __restrict__ E, const float* __restrict__ PA,
                                                     float* __restrict__ Wt, int64_t ldw, int64_t lda, int rows,
                                                     int s0, int s1, int t0, int t1)
{
    __shared__ __align__(16) float lds[UpdBlk::LDS_FLOATS];
    const int nbx = (t1 - t0 + 127) / 128;
    const unsigned p = xcd_group4(blockIdx.x, gridDim.x);
    const int bx = (int)(p % (unsigned)nbx), by = (int)(p / (unsigned)nbx);
    const int r = 128 * by, c = t0 + 128 * bx;
    const int rlim = min(128, rows - r), clim = min(128, t1 - c);
    Acc acc;
    acc_zero(acc);
    block_gemm<2, 2, RowK, RowK>(E + (int64_t)r * ldw, ldw, rlim, PA + (int64_t)c * lda, lda, clim, s0, s1, lds, acc);
    block_store<2, 2>(Wt + (int64_t)r * ldw + c, ldw, rlim, clim, -1.f, 1.f, acc);
}

// The same with one 64 x 64 output tile per workgroup (one 32 x 32 quadrant
// per wave), for small target ranges.
__global__ __launch_bounds__(256) void k_gptq_update_t(const float* __restrict__ E, const float* __restrict__ PA,
                                                       float* __restrict__ Wt, int64_t ldw, int64_t lda, int s0,
                                                       int s1, int t0)
{
    __shared__ __align__(16) float lds[kLds64];
    const int r = 64 * (int)blockIdx.y, c = t0 + 64 * (int)blockIdx.x;
    const int wave = threadIdx.x >> 6;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    block_gemm64<RowK, RowK>(E + (int64_t)r * ldw, ldw, PA + (int64_t)c * lda, lda, s0, s1, lds, acc);
    const int64_t rr = r + 32 * (wave >> 1), cc = c + 32 * (wave & 1);
    wave_store32(Wt + rr * ldw + cc, ldw, -1.f, 1.f, acc);
}

__global__ __launch_bounds__(256) void k_gptq_obj(const double* __restrict__ part, int64_t count,
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

// ------------------------------------------------------------ host side

namespace {

struct GptqPlan {
    int64_t m, n, Nt, Mp, Np, wgs;
    bool pad_a;
    size_t off_wt, off_e, off_obj, off_pa, total;
};

GptqPlan plan_gptq(int64_t m, int64_t n)
{
    GptqPlan p;
    p.m = m;
    p.n = n;
    p.Nt = ceil_div(n, kTile);
    p.Np = p.Nt * kTile;
    p.Mp = ceil_div(m, kGRows) * kGRows;
    p.wgs = p.Mp / kGRows;
    p.pad_a = (n % kTile) != 0;
    const size_t mat = sizeof(float) * (size_t)(p.Mp * p.Np);
    size_t off = 0;
    p.off_wt = off;
    off = align_up(off + mat);
    p.off_e = off;
    off = align_up(off + mat);
    p.off_obj = off;
    off = align_up(off + sizeof(double) * (size_t)(p.Nt * p.wgs));
    p.off_pa = 0;
    if (p.pad_a) {
        p.off_pa = off;
        off = align_up(off + sizeof(float) * (size_t)(p.Np * p.Np));
    }
    p.total = off;
    return p;
}

dim3 load_grid(int64_t R, int64_t C)
{
    return dim3((unsigned)ceil_div(C, 1024), (unsigned)std::min<int64_t>(R, 32768));
}

int load_vec(const float* src, int64_t lds) { return (lds % 4 == 0 && aligned16(src)) ? 1 : 0; }

struct GptqRun {
    SweepArgs sw;
    int Mp;
    int wgs;
    double* obj;
    hipStream_t s;
    Prof* prof;
};

// An update with fewer 128 x 128 blocks than this runs on 64 x 64 tiles.
constexpr int64_t kUpdBlockMin = 512;

void enqueue_update(GptqRun& R, int s0, int s1, int t0, int t1)
{
    const double rows = R.sw.m, K = s1 - s0, N = t1 - t0;
    const double fl = 2.0 * rows * K * N;
    const double by = 4.0 * (rows * K + N * K + 2.0 * rows * N);   // E, P_A block in; Wt read and written
    const int64_t blocks = ceil_div(R.Mp, 128) * ceil_div(t1 - t0, 128);
    if (blocks >= kUpdBlockMin) {
        launch(R.prof, KK_G_UPDATE, fl, by, k_gptq_update, dim3((unsigned)blocks), dim3(256), R.s,
               (const float*)R.sw.E, R.sw.PA, R.sw.Wt, R.sw.ldw, R.sw.lda, R.Mp, s0, s1, t0, t1);
    } else {
        launch(R.prof, KK_G_UPDATE_T, fl, by, k_gptq_update_t,
               dim3((unsigned)((t1 - t0) / 64), (unsigned)ceil_div(R.Mp, 64)), dim3(256), R.s, (const float*)R.sw.E,
               R.sw.PA, R.sw.Wt, R.sw.ldw, R.sw.lda, s0, s1, t0);
    }
}

void enqueue_sweep(GptqRun& R, int J)
{
    R.sw.J = J;
    if (R.obj) R.sw.objp = R.obj + (int64_t)J * R.wgs;
    // per row: the in-block triangular update (64 * 63 / 2 multiply-adds);
    // bytes: the Wt block and the P_A block in, E and V (+ err) out, codes
    const double rows = R.sw.m;
    const double fl = 2.0 * rows * (64.0 * 63.0 / 2.0);
    const double by = rows * 64.0 * (4.0 * (R.sw.err ? 4.0 : 3.0) + 1.0) + 4.0 * 64.0 * 64.0;
    launch(R.prof, KK_G_SWEEP, fl, by, k_gptq_sweep, dim3((unsigned)R.wgs), dim3(256), R.s, R.sw);
}

void gptq_rec(GptqRun& R, int J0, int J1)
{
    if (J1 - J0 == 1) {
        enqueue_sweep(R, J0);
        return;
    }
    const int mid = (J0 + J1) / 2;
    gptq_rec(R, J0, mid);
    enqueue_update(R, 64 * J0, 64 * mid, 64 * mid, 64 * J1);
    gptq_rec(R, mid, J1);
}

}  // namespace

size_t gptq_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0) return 0;
    const GptqPlan p = plan_gptq(ceil_div(m, 64) * 64, n);
    return p.total;
}

int gptq_enqueue(const float* W, int64_t m, int64_t n, const float* LA, const float* PA, const float* scale,
                 const float* zero, const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                 void* ws, hipStream_t s, Prof* prof, int64_t group_size)
{
    // Rows are padded to a multiple of 64 so that the 64 x 64 update tiles
    // stay inside the workspace; sweeps cover the same padded rows.
    const GptqPlan p = plan_gptq(ceil_div(m, 64) * 64, n);
    char* w = static_cast<char*>(ws);
    GptqRun R;
    R.prof = prof;
    R.s = s;
    SweepArgs& g = R.sw;
    g.Wt = reinterpret_cast<float*>(w + p.off_wt);
    g.E = reinterpret_cast<float*>(w + p.off_e);
    g.ldw = p.Np;
    const double dm = (double)m, dn = (double)n;
    if (p.pad_a) {
        float* pa = reinterpret_cast<float*>(w + p.off_pa);
        launch(prof, KK_G_LOAD, 0.0, 4.0 * (dn * dn + (double)(p.Np * p.Np)), k_gptq_load, load_grid(p.Np, p.Np),
               dim3(256), s, PA, n, n, n, pa, p.Np, p.Np, p.Np, load_vec(PA, n));
        g.PA = pa;
        g.lda = p.Np;
    } else {
        g.PA = PA;
        g.lda = n;
    }
    launch(prof, KK_G_LOAD, 0.0, 4.0 * (dm * dn + (double)(p.Mp * p.Np)), k_gptq_load, load_grid(p.Mp, p.Np),
           dim3(256), s, W, m, n, n, g.Wt, p.Mp, p.Np, p.Np, load_vec(W, n));
    if (hipGetLastError() != hipSuccess) return -1;
    g.scale = scale;
    g.zero = zero;
    g.maxq = maxq;
    g.gld = group_size > 0 ? ceil_div(n, group_size) : 1;
    g.gtiles = group_size > 0 ? (int)(group_size / kTile) : INT_MAX;
    g.m = (int)m;
    g.n = (int)n;
    g.codes = codes;
    g.V = V;
    g.err = err;
    g.LA = LA;
    g.objp = nullptr;
    g.vec_out = (n % kTile == 0 && (reinterpret_cast<uintptr_t>(codes) & 7u) == 0 && aligned16(V) &&
                 (err == nullptr || aligned16(err)))
                    ? 1
                    : 0;
    R.Mp = (int)p.Mp;
    R.wgs = (int)p.wgs;
    R.obj = objective ? reinterpret_cast<double*>(w + p.off_obj) : nullptr;
    gptq_rec(R, 0, (int)p.Nt);
    if (hipGetLastError() != hipSuccess) return -1;
    if (objective) {
        const double cnt = (double)(p.Nt * p.wgs);
        launch(prof, KK_G_OBJ, cnt, 8.0 * (cnt + 1.0), k_gptq_obj, dim3(1), dim3(256), s, (const double*)R.obj,
               p.Nt * p.wgs, objective);
        if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
}

}  // namespace bk
