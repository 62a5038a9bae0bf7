// solve.hip -- the BaKron rounding of W (m x n) under A (x) B, for gfx950.
//
// Method (paper summary "FastKron: Efficient Quantization with
// Kronecker-Factored Hessians", derivation naive -> antidiagonal -> BaKron,
// Theorem 3.2): GPTQ on vec(W) with Hessian A (x) B.  Quantizing entry (i, j)
// with raw error e changes only entries (i', j') with i' >= i and j' >= j, by
// e * P_B[i', i] * P_A[j', j] (P = L^-1 diag(L), L = RevCholesky).  So all
// entries of one anti-diagonal can be rounded together, and the anti-diagonal
// range can be split recursively: solve the first half, push its errors into
// the second half with dense products, then solve the second half.
//
// MI355X layout of that idea:
//  * 64 x 64 tiles.  Tile (I, J) only depends on tiles (I', J') with I' <= I,
//    J' <= J, so tile anti-diagonals K = I + J are the recursion's unit.
//  * Leaf (one launch per tile anti-diagonal, one workgroup per tile): the
//    tile and its diagonal P_A block sit in LDS; 127 in-tile anti-diagonal
//    steps quantize up to 64 entries each.  The value of entry (a, b) is
//        W~in[a,b] - sum_{a'<=a} P_B[a,a'] U[a',b],
//        U[a',b] = sum_{b'<=b, done} e[a',b'] P_A[b,b'],
//    two length-64 dot products per entry, split over 8 lanes and reduced
//    with lane shuffles (see k_leaf).
//  * Internal node (K0, mid, K1): stage 1 forms, per tile row I, the partial
//    products Y[I, J'] = sum_J E[I, J] P_A[J', J]^T over the source tiles
//    (K0 <= I + J < mid, J <= J'); stage 2 subtracts
//    sum_I P_B[I', I] Y[I, J'] from every target tile (mid <= I' + J' < K1).
//    Both are fp32 MFMA GEMMs whose K range follows the staircase of the
//    tile band.  A node of two leaves (K0, K0 + 1, K0 + 2) has no launch of
//    its own: the leaf of K0 + 1 applies both stages to its tile first
//    (leaf_prologue, which also serves wider nodes when kFold allows).
//  * On the upper levels a node's propagation is cut by target
//    anti-diagonal into parts with different due times; only the first is
//    on the caller's stream, the others run on library-owned streams beside
//    the latency-bound leaves (see the block schedule and enqueue_prop).
//
// Workspace (pitch Np = 64 * ceil(n / 64), Mp = 64 * ceil(m / 64)):
//   Wt  Mp x Np  working weights (W copied in, zero padded)
//   E   Mp x Np  raw errors of solved tiles
//   Y   Mp x Np  stage-1 partial products of unsplit nodes
//   Yd  Mp x Np  the same for the split nodes of depth d, one per depth
//   obj Mt x Nt  per-tile objective partials (double)
//   PAp Np x Np, PBp Mp x Mp  padded copies, only when n (m) is not a
//        multiple of 64.
//   sched  block lists of the propagation launches (k_sched)
// Padding entries are forced to zero error, so they never touch real ones.
#include <limits.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "gemm.hpp"
#include "internal.hpp"

namespace bk {

// Waves of the caller's stream's kernels (the leaves and the near parts of
// the propagation, the solve's critical path) take issue priority over the
// far parts' waves where the two share a CU.
#ifndef BAKRON_NEAR_PRIO
#define BAKRON_NEAR_PRIO 2
#endif
__device__ __forceinline__ void near_priority()
{
    if (BAKRON_NEAR_PRIO > 0) __builtin_amdgcn_s_setprio(BAKRON_NEAR_PRIO);
}

// dst (R x C, pitch ldd) = src (rows x cols, pitch lds) with zeros outside.
// C and ldd are multiples of 4: each thread writes four adjacent columns
// with one 16-byte store, reading them with one 16-byte load where they lie
// inside src and src's rows are 16-byte aligned (vec).
__global__ __launch_bounds__(256) void k_copy_pad(const float* __restrict__ src, int64_t rows, int64_t cols,
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

struct LeafArgs {
    float* Wt;            // Mp x Np working weights (pitch ldw)
    float* E;             // Mp x Np raw errors (pitch ldw)
    int64_t ldw;
    const float* PA;      // P_A (pitch lda)
    int64_t lda;
    const float* PB;      // P_B (pitch ldb)
    int64_t ldb;
    const float* scale;   // grid of row i, tile column J: index i * gld + J / gtiles
    const float* zero;
    const int32_t* maxq;
    int64_t gld;          // grid pitch: 1 (per row) or the number of column groups
    int gtiles;           // tiles per column group (group size / 64; huge for per-row grids)
    int m, n;
    uint8_t* codes;       // m x n outputs (pitch n)
    float* V;
    float* err;           // nullable
    const float* LA;      // nullable: diag source for the objective (pitch n)
    const float* LB;      // nullable (pitch m)
    double* objp;         // nullable: Mt x Nt partials
    int Nt;
    int K;                // tile anti-diagonal
    int I_lo;             // first tile row on it
    int nsrc;             // > 0: the leaf first applies the errors of anti-diagonals K - nsrc .. K - 1 (a narrow node's)
    int vec_out;          // outputs may use 16-byte stores
};

constexpr int kLP = 68;   // LDS pitch (floats) of the P_A, U^T and E tiles

// Lane shuffles inside a row's group of 8 lanes (two quads of a 16-lane DPP
// row), all DPP moves (no LDS round trip).
// value of lane 0 of the group, in every lane of the group
__device__ __forceinline__ float bcast8_lane0(float x)
{
    const int b = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x00, 0xF, 0xF, false);   // quad_perm [0,0,0,0]
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x114, 0xF, 0xA, false));  // quads 1, 3 <- 0, 2
}

// sum over the 8 lanes of the group, in every lane
__device__ __forceinline__ float sum8(float x)
{
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
    x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, true));
    const int xi = __builtin_bit_cast(int, x);
    int y = __builtin_amdgcn_update_dpp(0, xi, 0x104, 0xF, 0x5, false);   // quads 0, 2 <- 1, 3 (row_shl:4)
    y = __builtin_amdgcn_update_dpp(y, xi, 0x114, 0xF, 0xA, false);       // quads 1, 3 <- 0, 2 (row_shr:4)
    return x + __builtin_bit_cast(float, y);
}

// One tile (I, J) of tile anti-diagonal K per workgroup; 512 threads = 64
// rows x 8 lanes (each lane owns 8 of the 64 columns of a row), so that two
// waves share each SIMD and hide each other's latencies.
//
// In-tile step d visits entry (a, b = d - a) of every row a.  Its value is
//   w~ = W~in[a,b] - pu - ps,
//   pu = sum_{c<b} e[a,c] P_A[b,c]          (own row, earlier columns)
//   ps = sum_{r<a} P_B[a,r] U[r,b],  U[r,b] = sum_{c<=b} e[r,c] P_A[b,c]
// (P_A, P_B: the diagonal blocks of this tile).
//  * pu is accumulated forward: each row keeps U[a, b .. b+63] (only the
//    errors found so far) in registers, 8 columns per lane, in a window that
//    starts at the row's current column b.  After rounding (a, b) the row adds
//    e[a,b] P_A[c,b] to every column c of the window, reading P_A[b .. b+63, b]
//    from the skewed copy S[b][j] = P_A[b+j, b] (two 16-byte reads per lane);
//    the window then moves on by one column.  The loop is unrolled 8 times
//    so that the move is a renaming of registers, plus one lane shift for
//    the column passed between neighbouring lanes.  The window's first
//    column is pu for the next step, and at the diagonal P_A[b,b] = 1 makes
//    it U[a,b] = pu + e[a,b].
//  * ps is gathered from U^T in LDS: each step reads column b+1 of U^T
//    (rows r < a-1, final one step earlier) for the next step, and the one
//    new term, U[a-1,b], is read at the start of the step.
// The critical path of a step is: barrier, read U[a-1,b], one FMA, round,
// write e[a,b] and U[a,b], barrier.

struct LeafRow {
    const float* sW;
    const float* sZ;   // 8 zeros: the operand of lanes whose reads could only return zeros
    const float* sS;
    float* sUT;
    float* sF;
    uint8_t* sC;
    int a, sg, am1;
    float sc, sinv, zc, mq, pbm1;
    bool row_ok;
    int64_t c0;
    int n;
};

template <int U>
__device__ __forceinline__ void leaf_step(const LeafRow& L, int d0, float (&R)[8], const float (&pbz)[8], float& pu,
                                          float& psp, float& wcur)
{
    const int d = d0 + U;
    const int b = d - L.a, bn = b + 1;
    const bool act = (unsigned)b < 64u;
    const bool actn = (unsigned)bn < 64u;
    // clamped, in-bounds indices; what inactive rows read is masked below
    const int bc = min(max(b, 0), 63), bnc = min(max(bn, 0), 63);
    const float fresh = L.sUT[bc * kLP + L.am1];   // U[a-1][b]
    const float wnext = L.sW[L.a * 64 + bnc];
    __builtin_amdgcn_sched_barrier(0);             // the fresh value first
    // S[b][8 sg ..] is zero past the tile (8 sg > 63 - b) and U[8 sg ..][b + 1]
    // only enters for rows below a - 1: such lanes read the shared zeros
    // instead, which the LDS serves as one broadcast
    const bool need_ps = actn && 8 * L.sg < L.a - 1;
    const float* sp = (act && 8 * L.sg <= 63 - b) ? L.sS + bc * kLP + 8 * L.sg : L.sZ;   // P_A[b + 8 sg + i][b]
    const float* up = need_ps ? L.sUT + bnc * kLP + 8 * L.sg : L.sZ;                    // U[8 sg + i][b + 1]
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(sp);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(sp + 4);
    const f32x4 u0 = *reinterpret_cast<const f32x4*>(up);
    const f32x4 u1 = *reinterpret_cast<const f32x4*>(up + 4);
    // critical path: this step's entry
    const float ps = psp + L.pbm1 * fresh;         // pbm1 == 0 on row 0
    const float w = wcur - pu - ps;
    // w / sc correctly rounded (Markstein: with y = RN(1/sc), q0 = RN(w y)
    // is within an ulp, the remainder w - sc q0 is exact under fma, and
    // RN(q0 + r y) is RN(w / sc)); then x = RN(q + zc) as in the oracle.
    float q0 = w * L.sinv;
    const float rem = fmaf(-q0, L.sc, w);
    q0 = fmaf(rem, L.sinv, q0);
    const float x = q0 + L.zc;
    const float c = fminf(fmaxf(rintf(x), 0.f), L.mq);
    const float v = L.sc * (c - L.zc);
    const bool ok = act && L.row_ok && (L.c0 + b) < L.n;
    const float e = ok ? (w - v) : 0.f;
    if (act && L.sg == 0) {
        L.sF[L.a * kLP + b] = e;
        L.sUT[b * kLP + L.a] = pu + e;
        L.sC[L.a * 64 + b] = ok ? (uint8_t)c : (uint8_t)0;
    }
    // window update: logical column k (= b + 8 sg + k) lives in R[(k + U) & 7]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        R[(k + U) & 7] = fmaf(e, s0[k], R[(k + U) & 7]);
        R[(k + 4 + U) & 7] = fmaf(e, s1[k], R[(k + 4 + U) & 7]);
    }
    // next step's ps without the fresh term (P_B[a][a-1] is zero in pbz)
    float t0 = pbz[0] * u0.x, t1 = pbz[1] * u0.y;
    t0 = fmaf(pbz[2], u0.z, t0);
    t1 = fmaf(pbz[3], u0.w, t1);
    t0 = fmaf(pbz[4], u1.x, t0);
    t1 = fmaf(pbz[5], u1.y, t1);
    t0 = fmaf(pbz[6], u1.z, t0);
    t1 = fmaf(pbz[7], u1.w, t1);
    const float psn = sum8(t0 + t1);   // lanes without rows r < a - 1 read the zero block
    // move the window one column on: logical 0 (column b, done) becomes
    // logical 7 and takes the next lane's logical 0 (column b + 8 (sg + 1)).
    // For the row's last lane (sg = 7) that is column b + 64: lane 7 of an
    // even row takes the next row's lane 0 and the last lane of a DPP row
    // keeps its own value.  Either way the value is past the tile for a row
    // that has started, and zero for one that has not (so is the next row's
    // whole window then), so no lane needs masking.
    constexpr int P0 = U & 7;
    R[P0] = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, R[P0]),
                                                                  __builtin_bit_cast(int, R[P0]), 0x101, 0xF, 0xF,
                                                                  false));   // row_shl:1
    // pu of the next step: logical 0 of lane 0 of the row's group
    const float pun = bcast8_lane0(R[(U + 1) & 7]);
    // unconditional: a row that has not started reads clamped (real)
    // operands and gets pu = 0 (no errors yet), psp = 0 (no U reads) and some
    // W~ value, all set again at the step before its first column; a finished
    // row's values are not used
    pu = pun;
    psp = psn;
    wcur = wnext;
    __syncthreads();
}

// A narrow node's propagation, applied by its leaves.  A node of at most
// kFold anti-diagonals [K0, K1) has no propagation launches: the leaf of
// anti-diagonal K in it first applies, to each of its tiles (It, Jt), the
// errors of the node's earlier anti-diagonals [K0, K) = [K - nsrc, K):
//   Y_I = sum_J E[I, J] P_A[Jt, J]^T        (stage 1; J <= Jt, I + J in [K - nsrc, K))
//   W~[It, Jt] -= sum_I P_B[It, I] Y_I       (stage 2, I = It - nsrc .. It ascending)
// Errors of anti-diagonals before K0 reached W~ through the propagation of
// the nodes above.  Rows are taken two at a time: stage 1 of a row on four
// waves (one 32 x 32 quadrant each; the row's source tiles accumulated in
// ascending order), its Y tile in LDS (sY0, sY1: 64 x kLP each), then stage
// 2 of both rows on the first four waves, accumulating in registers.
// Fragments come straight from global memory; Y is rounded as the tile
// kernels store it (with one source tile per row, nsrc = 1, the result is
// theirs bit for bit).  The updated tile lands in sW, the leaf's copy.
__device__ __forceinline__ void leaf_prologue(const LeafArgs& g, int It, int Jt, float* __restrict__ sY0,
                                              float* __restrict__ sY1, float* __restrict__ sW)
{
    const int K = g.K, ns = g.nsrc;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, quad = wave & 3;
    const int ml = lane & 31, kl = 4 * (lane >> 5);
    const int ra = 32 * (quad >> 1) + ml, rb = 32 * (quad & 1) + ml;
    const int Ilo = max(0, It - ns), Ihi = min(It, K - 1);   // rows with a source tile J <= Jt
    f32x16 acc2;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc2[r] = 0.f;
    for (int I0 = Ilo; I0 <= Ihi; I0 += 2) {
        const int I = I0 + (wave >> 2);
        if (I <= Ihi) {
            const int jlo = max(0, K - ns - I), jhi = min(K - 1 - I, Jt);
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
            for (int J = jlo; J <= jhi; ++J) {
                const float* a0 = g.E + (int64_t)I * 64 * g.ldw + (int64_t)J * 64;
                const float* b0 = g.PA + (int64_t)Jt * 64 * g.lda + (int64_t)J * 64;
                f32x4 a[8], b[8];
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    a[st] = *reinterpret_cast<const f32x4*>(a0 + (int64_t)ra * g.ldw + 8 * st + kl);
                    b[st] = *reinterpret_cast<const f32x4*>(b0 + (int64_t)rb * g.lda + 8 * st + kl);
                }
#pragma unroll
                for (int st = 0; st < 8; ++st)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[st][q], b[st][q], acc, 0, 0, 0);
            }
            float* y = (I == I0 ? sY0 : sY1) + 32 * (quad >> 1) * kLP + 32 * (quad & 1);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float one = 1.f, none = 0.f;   // as stage 1 stores Y: 1 acc + 0 0
                y[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kLP + ml] = one * acc[r] + none * none;
            }
        }
        __syncthreads();
        if (wave < 4) {
            for (int Is = I0; Is <= min(I0 + 1, Ihi); ++Is) {
                const float* a0 = g.PB + (int64_t)It * 64 * g.ldb + (int64_t)Is * 64;
                const float* y = (Is == I0 ? sY0 : sY1) + rb;
                f32x4 a[8];
#pragma unroll
                for (int st = 0; st < 8; ++st)
                    a[st] = *reinterpret_cast<const f32x4*>(a0 + (int64_t)ra * g.ldb + 8 * st + kl);
#pragma unroll
                for (int st = 0; st < 8; ++st) {
                    const float* c = y + (8 * st + kl) * kLP;
                    const f32x4 bv = {c[0], c[kLP], c[2 * kLP], c[3 * kLP]};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[st][q], bv[q], acc2, 0, 0, 0);
                }
            }
        }
        __syncthreads();   // the Y tiles are read before the next rows (or the leaf) overwrite them
    }
    if (wave < 4) {
        // W~ - acc, as the tile kernels' epilogue forms it (alpha acc + beta old)
        const float* wq = g.Wt + ((int64_t)It * 64 + 32 * (quad >> 1)) * g.ldw + (int64_t)Jt * 64 + 32 * (quad & 1);
        float* sq = sW + 32 * (quad >> 1) * 64 + 32 * (quad & 1);
        const float alpha = -1.f, beta = 1.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            sq[row * 64 + ml] = alpha * acc2[r] + beta * wq[(int64_t)row * g.ldw + ml];
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(512) void k_leaf(LeafArgs g)
{
    near_priority();
    __shared__ float sW[64 * 64];
    // sS and sUT hold the Y tiles of a narrow node's propagation first
    __shared__ __align__(16) float sS[64 * kLP];    // sS[b][j] = P_A[b + j][b], zero past the tile
    __shared__ __align__(16) float sUT[64 * kLP];   // sUT[b][a] = U[a][b]
    __shared__ __align__(16) float sF[64 * kLP];    // raw errors e[a][b]
    __shared__ __align__(16) uint8_t sC[64 * 64];
    __shared__ __align__(16) float sZ[8];
    __shared__ double sRed[8];

    const int I = g.I_lo + blockIdx.x;
    const int J = g.K - I;
    const int t = threadIdx.x;
    const int a = t >> 3, sg = t & 7;
    if (t < 8) sZ[t] = 0.f;
    const int64_t r0 = (int64_t)I * 64, c0 = (int64_t)J * 64;
    if (g.nsrc) leaf_prologue(g, I, J, sS, sUT, sW);

    for (int idx = t; idx < 64 * kLP; idx += 512) {
        sS[idx] = 0.f;
        sUT[idx] = 0.f;
        sF[idx] = 0.f;
    }
    f32x4 pa[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int f = t + 512 * u;
        const int row = f >> 4, cq = 4 * (f & 15);
        if (!g.nsrc) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(g.Wt + (r0 + row) * g.ldw + c0 + cq);
            *reinterpret_cast<f32x4*>(sW + row * 64 + cq) = w;
        }
        pa[u] = *reinterpret_cast<const f32x4*>(g.PA + (c0 + row) * g.lda + c0 + cq);
    }
    __syncthreads();   // zeroing done before the skewed scatter
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int f = t + 512 * u;
        const int row = f >> 4, cq = 4 * (f & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (row >= cq + i) sS[(cq + i) * kLP + (row - cq - i)] = pa[u][i];   // P_A[row][col], col <= row
    }
    // P_B row a, this lane's 8 columns; pbz drops column a-1 (the fresh term)
    float pbz[8];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(g.PB + (r0 + a) * g.ldb + r0 + 8 * sg + 4 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) pbz[4 * q + i] = (8 * sg + 4 * q + i == a - 1) ? 0.f : v[i];
    }
    const int64_t grow = r0 + a;
    LeafRow L;
    L.sW = sW;
    L.sZ = sZ;
    L.sS = sS;
    L.sUT = sUT;
    L.sF = sF;
    L.sC = sC;
    L.a = a;
    L.sg = sg;
    L.am1 = a > 0 ? a - 1 : 0;
    L.pbm1 = a > 0 ? g.PB[(r0 + a) * g.ldb + r0 + a - 1] : 0.f;   // P_B[a][a-1]
    L.row_ok = grow < g.m;
    const int gcol = J / g.gtiles;   // this tile's column group (every column of a tile is in one group)
    const int64_t gi = grow * g.gld + gcol;
    L.sc = L.row_ok ? g.scale[gi] : 1.f;
    L.zc = L.row_ok ? g.zero[gi] : 0.f;
    L.mq = L.row_ok ? (float)g.maxq[gi] : 0.f;
    L.sinv = 1.f / L.sc;   // correctly rounded
    L.c0 = c0;
    L.n = g.n;
    __syncthreads();

    float R[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) R[k] = 0.f;
    float pu = 0.f, psp = 0.f;
    float wcur = (a == 0) ? sW[0] : 0.f;
    // 127 steps, in 16 unrolled groups of 8 (the 128th step is idle for every row)
    for (int d0 = 0; d0 < 128; d0 += 8) {
        leaf_step<0>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<1>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<2>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<3>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<4>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<5>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<6>(L, d0, R, pbz, pu, psp, wcur);
        leaf_step<7>(L, d0, R, pbz, pu, psp, wcur);
    }

    // Outputs: raw errors to the workspace, codes / values / errors to the
    // caller, and this tile's objective partial.  Thread (row, 8 columns).
    const int row = t >> 3, cs = 8 * (t & 7);
    const int64_t orow = r0 + row;
    double objs = 0.0;
    const float lb = (g.objp && orow < g.m) ? g.LB[orow * g.m + orow] : 0.f;
#pragma unroll
    for (int q = 0; q < 2; ++q)
        *reinterpret_cast<f32x4*>(g.E + orow * g.ldw + c0 + cs + 4 * q) =
            *reinterpret_cast<const f32x4*>(sF + row * kLP + cs + 4 * q);
    if (orow < g.m) {
        const float so = g.scale[orow * g.gld + gcol], zo = g.zero[orow * g.gld + gcol];
        if (g.vec_out) {
            *reinterpret_cast<uint2*>(g.codes + orow * g.n + c0 + cs) =
                *reinterpret_cast<const uint2*>(sC + row * 64 + cs);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                f32x4 v;
                v.x = so * ((float)sC[row * 64 + cs + 4 * q + 0] - zo);
                v.y = so * ((float)sC[row * 64 + cs + 4 * q + 1] - zo);
                v.z = so * ((float)sC[row * 64 + cs + 4 * q + 2] - zo);
                v.w = so * ((float)sC[row * 64 + cs + 4 * q + 3] - zo);
                *reinterpret_cast<f32x4*>(g.V + orow * g.n + c0 + cs + 4 * q) = v;
                if (g.err)
                    *reinterpret_cast<f32x4*>(g.err + orow * g.n + c0 + cs + 4 * q) =
                        *reinterpret_cast<const f32x4*>(sF + row * kLP + cs + 4 * q);
            }
        } else {
            for (int k = 0; k < 8; ++k) {
                const int64_t col = c0 + cs + k;
                if (col >= g.n) break;
                const uint8_t c = sC[row * 64 + cs + k];
                g.codes[orow * g.n + col] = c;
                g.V[orow * g.n + col] = so * ((float)c - zo);
                if (g.err) g.err[orow * g.n + col] = sF[row * kLP + cs + k];
            }
        }
        if (g.objp) {
            for (int k = 0; k < 8; ++k) {
                const int64_t col = c0 + cs + k;
                if (col >= g.n) break;
                const double q = (double)lb * (double)g.LA[col * g.n + col] * (double)sF[row * kLP + cs + k];
                objs += q * q;
            }
        }
    }
    if (g.objp) {
        for (int off = 32; off > 0; off >>= 1) objs += __shfl_xor(objs, off);
        if ((t & 63) == 0) sRed[t >> 6] = objs;
        __syncthreads();
        if (t == 0) {
            double sum = 0.0;
            for (int w = 0; w < 8; ++w) sum += sRed[w];
            g.objp[(int64_t)I * g.Nt + J] = sum;
        }
    }
}

// ------------------------------------------------------ propagation

// Workgroups are dealt to the eight XCDs round-robin (workgroup p runs on
// XCD p % 8), each XCD with its own L2.  Consecutive list entries share
// most of their operands (the same block column of neighbouring rows), so
// groups of kXcdGroup consecutive entries are sent to one XCD: within each
// run of 8 * kXcdGroup workgroups, p -> entry (p % 8) * kXcdGroup + p / 8.
// The longest-first order survives at the granularity of a run.
#ifndef BAKRON_XCD_GROUP
#define BAKRON_XCD_GROUP 4
#endif
constexpr int kXcdGroup = BAKRON_XCD_GROUP;

// The 64 x 64 tile kernels of the small nodes can map their work items the
// same way (consecutive items share an operand strip: the error strip of a
// tile row in stage 1, the Y strip of a tile column in stage 2).
#ifndef BAKRON_T_XCD
#define BAKRON_T_XCD 0
#endif
constexpr bool kTileXcd = BAKRON_T_XCD != 0;

__device__ __forceinline__ unsigned xcd_entry(unsigned p, unsigned n)
{
    constexpr unsigned run = 8u * kXcdGroup;
    if (p >= n / run * run) return p;   // ragged last run: identity
    const unsigned r = p % run;
    return p - r + (r % 8u) * kXcdGroup + r / 8u;
}

typedef Gemm<1, 4, RowK, RowK> RowBlk;   // stage 1: 64 rows (one tile row) x 256 cols
typedef Gemm<4, 1, RowK, KRow> ColBlk;   // stage 2: 256 rows x 64 cols (one tile column)

// ------------------------------------------------------ block schedule
//
// A propagation block's K extent follows the staircase of the tile band, so
// the blocks of one launch differ in length by up to two orders of
// magnitude; started in plain index order, the long ones start late and the
// launch ends with most CUs idle.  k_sched writes, for every internal node
// of the recursion, each of its two stages and each part (below), the
// blocks sorted by decreasing K extent (longest first), and the propagation
// kernels take their block from that list.  The order only decides which CU
// computes which block: every block writes its own outputs, so results do
// not depend on it.
//
// Nodes are numbered as in a heap: the root [0, Kt) is (depth 0, pos 0) and
// node (d, p) = [K0, K1) has children (d + 1, 2p) = [K0, mid) and
// (d + 1, 2p + 1) = [mid, K1), mid = (K0 + K1) / 2.  A node at depth d is at
// most w_d = ceil(Kt / 2^d) anti-diagonals wide, so a stage has at most
// max(Mt, Nt) * ceil(w_d / 4) blocks: that is the list capacity cap[d], and
// the list of (d, p, stage, part) starts at
// base[d] + (kNodeLists p + kMaxParts stage + part) * cap[d], the early
// pass's (below) at base[d] + (kNodeLists p + 2 kMaxParts) * cap[d].
// An entry packs (tile row or column) << 16 | block index.
//
// Parts.  The right child [mid, K1) of a node first solves [mid, m2),
// m2 = (mid + K1) / 2, which needs only the node's updates of the target
// anti-diagonals [mid, m2) (the near part).  The updates of [m2, K1) (the
// far part) are not needed before the right child's own propagation, so on
// the upper levels (depth < split_depth, K1 - mid >= kSplitMin) the far
// part runs on a second stream while [mid, m2) is being solved.  Stage 1 of
// the near part forms Y[I, J'] for J' < m2 - I (what near targets read),
// the far part the remaining columns J' < K1 - I; far targets read both.
// An unsplit node is one part: targets [mid, K1), Y columns J' < K1 - I.
//
// Early sources.  Stage 1 of an upper node sums over the source tiles of
// [K0, mid), but those of [K0, q), q = (K0 + mid) / 2 (the left child's
// split point), are final once [K0, q) is solved, long before mid.  So on
// the upper levels (depth < early_depth, left child at least kEarlyMin
// wide, right child at least kSplitMin wide: the split nodes) stage 1 runs
// in two source passes: the early pass forms Y[I, J'] over the sources
// [K0, q) for every Y column of the node (J' < K1 - I), on the depth's own
// stream as soon as [K0, q) is solved; the node's parts then add the
// sources [q, mid) to it (Y = late + early on rows I < q, which hold early
// sources).  The near part on the caller's stream is left with the late
// sources only.  Where a node is not split (bakron_solve_batch, the
// allocation-free entry point, no library stream) the same two passes run
// in place on the caller's stream, so every schedule rounds alike.

constexpr int kMaxDepth = 12;                 // Kt <= 2047 needs 11 levels of internal nodes
constexpr int kMaxKTiles = kMaxDim / kTile;   // K extent of a block, in tiles
#ifndef BAKRON_SPLIT_DEPTH
#define BAKRON_SPLIT_DEPTH 4
#endif
constexpr int kSplitDepth = BAKRON_SPLIT_DEPTH;   // nodes above this depth may be split
static_assert(kSplitDepth <= kSideSlots, "one library stream per split depth");
#ifndef BAKRON_SPLIT3_DEPTH
#define BAKRON_SPLIT3_DEPTH 3
#endif
constexpr int kSplit3Depth = BAKRON_SPLIT3_DEPTH;  // nodes above this depth may be cut in more than two
#ifndef BAKRON_MAX_PARTS
#define BAKRON_MAX_PARTS 3
#endif
constexpr int kMaxParts = BAKRON_MAX_PARTS;
#ifndef BAKRON_SPLIT_MIN
#define BAKRON_SPLIT_MIN 8
#endif
constexpr int kSplitMin = BAKRON_SPLIT_MIN;       // ... when the right child is at least this wide
#ifndef BAKRON_EARLY_DEPTH
#define BAKRON_EARLY_DEPTH 1
#endif
constexpr int kEarlyDepth = BAKRON_EARLY_DEPTH;   // nodes above this depth may take an early source pass
#ifndef BAKRON_EARLY_MIN
#define BAKRON_EARLY_MIN 8
#endif
constexpr int kEarlyMin = BAKRON_EARLY_MIN;       // ... when the left child is at least this wide
static_assert(kEarlyMin >= 4, "the left child of an early node has a left child of its own");
#ifndef BAKRON_EARLY_GRID
#define BAKRON_EARLY_GRID 192
#endif
constexpr unsigned kEarlyGrid = BAKRON_EARLY_GRID;   // workgroups of an early pass on a library stream
// block lists per node: (stage, part) at kMaxParts stage + part, then the early pass
constexpr int kNodeLists = 2 * kMaxParts + 1;

struct SchedGeom {
    int Mt, Nt, Kt, levels;
    int split_depth;    // nodes above this depth may be cut in parts (0: none)
    int split3_depth;   // ... and in up to kMaxParts parts above this one
    int early_depth;    // nodes above this depth may take an early source pass (not changed by unsplit runs)
    int64_t base[kMaxDepth];
    int64_t cap[kMaxDepth];
};

// Whether node (d, [K0, K1)) forms stage 1 in an early and a late source
// pass (split at (K0 + mid) / 2).
__host__ __device__ inline bool node_early(const SchedGeom& g, int d, int K0, int mid, int K1)
{
    return d < g.early_depth && mid - K0 >= kEarlyMin && K1 - mid >= kSplitMin;
}

// Parts of node (d, [K0, K1)): 1 (unsplit), 2 (targets [mid, m2) and
// [m2, K1)) or 3 (the first of those cut again at m3 = (mid + m2) / 2, the
// split point of the right child's left child).
__host__ __device__ inline int node_parts(const SchedGeom& g, int d, int mid, int K1)
{
    if (d >= g.split_depth || K1 - mid < kSplitMin) return 1;
    int parts = 2, b = (mid + K1) / 2;
    while (parts < kMaxParts && d < g.split3_depth && b - mid >= kSplitMin) {
        b = (mid + b) / 2;
        ++parts;
    }
    return parts;
}

// Part `part` of a node cut into `parts`: it forms the stage-1 Y columns
// y0 - I <= J' < y1 - I (the first part from the first source column) and
// updates the target anti-diagonals [t0, t1).  The cuts are the split
// points down the left spine of the right child: K1, m2 = (mid + K1) / 2,
// (mid + m2) / 2, ...
struct PartRange {
    int y0, y1, t0, t1;
    __host__ __device__ PartRange(int parts, int part, int K0, int mid, int K1)
    {
        int hi = K1, lo = parts > 1 ? (mid + K1) / 2 : mid;   // part parts - 1 is [lo, hi)
        for (int k = parts - 1; k > part; --k) {
            hi = lo;
            lo = k - 1 > 0 ? (mid + lo) / 2 : mid;
        }
        t0 = lo;
        t1 = hi;
        y0 = part == 0 ? K0 : t0;
        y1 = t1;
    }
};

// Stage 1 block (row I, block b): target columns j0 = tl + 4b .. jh, source
// columns sl .. min(sh, jh).  y0 is where this part's Y columns start
// (a far part skips the columns its near part formed).
struct RowSpan {
    int sl, sh, tl, th;
    __host__ __device__ RowSpan(int I, int K0, int mid, int y0, int y1, int Nt)
        : sl(max(0, K0 - I)), sh(min(Nt - 1, mid - 1 - I)), tl(max(max(0, K0 - I), y0 - I)),
          th(min(Nt - 1, y1 - 1 - I)) {}
    __host__ __device__ int blocks() const { return max(0, (th - tl + 4) / 4); }
    __host__ __device__ int ktiles(int b) const { return min(sh, min(th, tl + 4 * b + 3)) - sl + 1; }
};

// Stage 2 block (column J, block b): target rows i0 = tl + 4b .. ih on the
// target anti-diagonals [t0, t1), source rows slo .. min(mid - 1, ih).
struct ColSpan {
    int tl, th, slo, mid;
    __host__ __device__ ColSpan(int J, int K0, int mid_, int t0, int t1, int Mt)
        : tl(max(0, t0 - J)), th(min(Mt - 1, t1 - 1 - J)), slo(max(0, K0 - J)), mid(mid_) {}
    __host__ __device__ int blocks() const { return max(0, (th - tl + 4) / 4); }
    __host__ __device__ int ktiles(int b) const { return min(mid - 1, min(th, tl + 4 * b + 3)) - slo + 1; }
};

__host__ __device__ inline int rows_lo(int K0, int Nt) { return max(0, K0 - (Nt - 1)); }
__host__ __device__ inline int rows_hi(int mid, int Mt) { return min(Mt - 1, mid - 1); }
__host__ __device__ inline int cols_lo(int t0, int Mt) { return max(0, t0 - (Mt - 1)); }
__host__ __device__ inline int cols_hi(int t1, int Nt) { return min(Nt - 1, t1 - 1); }

// One workgroup per (heap slot, stage, part): counting sort of the part's
// blocks by K extent, descending.  Stage 2 is the early source pass (part 0
// only): stage 1 over the sources [K0, q) and every Y column of the node;
// stage 1 of an early node's parts then takes the sources [q, mid).
__global__ __launch_bounds__(256) void k_sched(SchedGeom g, uint32_t* __restrict__ out)
{
    __shared__ int cnt[kMaxKTiles + 1];
    __shared__ int kmax;
    const int t = threadIdx.x;
    const unsigned slot = blockIdx.x + 1u;
    const int d = 31 - __builtin_clz(slot);
    const int p = (int)(slot - (1u << d));
    const int stage = blockIdx.y, part = blockIdx.z;
    int K0 = 0, K1 = g.Kt;
    for (int l = d - 1; l >= 0; --l) {
        if (K1 - K0 < 2) return;          // no node at this slot
        const int mid = (K0 + K1) / 2;
        if ((p >> l) & 1) K0 = mid; else K1 = mid;
    }
    if (K1 - K0 < 2) return;              // a leaf: nothing to propagate
    const int mid = (K0 + K1) / 2;
    const int parts = node_parts(g, d, mid, K1);
    if (part >= parts) return;
    const bool early = node_early(g, d, K0, mid, K1);
    if (stage == 2 && (!early || part > 0)) return;
    const PartRange pr(parts, part, K0, mid, K1);
    // the stage-1 pass this list is for: sources [sk0, smid), Y columns [y0, y1)
    const int q = (K0 + mid) / 2;
    const int sk0 = stage == 2 ? K0 : (early ? q : K0), smid = stage == 2 ? q : mid;
    const int y0 = stage == 2 ? K0 : pr.y0, y1 = stage == 2 ? K1 : pr.y1;
    uint32_t* list = out + g.base[d] + (int64_t)(kNodeLists * p + kMaxParts * stage + part) * g.cap[d];
    const bool rows = stage != 1;
    const int lo = rows ? rows_lo(sk0, g.Nt) : cols_lo(pr.t0, g.Mt);
    const int hi = rows ? rows_hi(smid, g.Mt) : cols_hi(pr.t1, g.Nt);

    for (int k = t; k <= kMaxKTiles; k += 256) cnt[k] = 0;
    if (t == 0) kmax = 0;
    __syncthreads();
    int km = 0;
    for (int u = lo + t; u <= hi; u += 256) {
        if (rows) {
            const RowSpan s(u, sk0, smid, y0, y1, g.Nt);
            for (int b = 0; b < s.blocks(); ++b) {
                const int k = s.ktiles(b);
                atomicAdd(&cnt[k], 1);
                km = max(km, k);
            }
        } else {
            const ColSpan s(u, K0, mid, pr.t0, pr.t1, g.Mt);
            for (int b = 0; b < s.blocks(); ++b) {
                const int k = s.ktiles(b);
                atomicAdd(&cnt[k], 1);
                km = max(km, k);
            }
        }
    }
    atomicMax(&kmax, km);
    __syncthreads();
    if (t == 0) {   // exclusive prefix sum from the longest extent down
        int run = 0;
        for (int k = kmax; k >= 1; --k) {
            const int c = cnt[k];
            cnt[k] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int u = lo + t; u <= hi; u += 256) {
        if (rows) {
            const RowSpan s(u, sk0, smid, y0, y1, g.Nt);
            for (int b = 0; b < s.blocks(); ++b) list[atomicAdd(&cnt[s.ktiles(b)], 1)] = ((uint32_t)u << 16) | (uint32_t)b;
        } else {
            const ColSpan s(u, K0, mid, pr.t0, pr.t1, g.Mt);
            for (int b = 0; b < s.blocks(); ++b) list[atomicAdd(&cnt[s.ktiles(b)], 1)] = ((uint32_t)u << 16) | (uint32_t)b;
        }
    }
}

// ------------------------------------------------------ propagation

// Stage 1 of node (K0, mid, K1), one part: block (row I, b) from the
// schedule computes, for the (up to) four target tile columns J' = j0 .. jh
// of its part,
//   Y[I, J'] = sum_{J = sl .. min(sh, J')} E[I, J] P_A[J', J]^T.
// P_A[J', J] is zero for J > J', so the block uses K = sl .. min(sh, jh).
// A late source pass is launched with K0 = q; on its rows I < acc_rows
// (= q) it adds the early pass's Y instead of storing over it.
//
// A launch covers `count` list entries with gridDim.x <= count workgroups,
// each taking entries blockIdx.x, blockIdx.x + gridDim.x, ... (a far part
// runs on a capped grid, next to the leaves; see enqueue_prop).  Every
// kernel has a `_far` twin, used for the far parts, so that timings of the
// two kinds of launch are told apart: the same body, except for this stage's
// block kernel, whose far twin takes two blocks per workgroup (same blocks,
// same results).
__device__ __forceinline__ void prop_rows_body(const float* __restrict__ E, const float* __restrict__ PA,
                                               float* __restrict__ Y, int64_t ldw, int64_t lda,
                                               int K0, int mid, int y0, int y1, int Mt, int Nt,
                                               const uint32_t* __restrict__ list, unsigned count, int acc_rows)
{
    __shared__ __align__(16) float lds[RowBlk::LDS_FLOATS];
    for (unsigned q = blockIdx.x; q < count; q += gridDim.x) {
        const uint32_t e = list[xcd_entry(q, count)];
        const int I = (int)(e >> 16), b = (int)(e & 0xffffu);
        if (I < rows_lo(K0, Nt) || I > rows_hi(mid, Mt)) continue;
        const RowSpan s(I, K0, mid, y0, y1, Nt);
        const int j0 = s.tl + 4 * b;
        if (j0 > s.th) continue;
        const int jh = min(s.th, j0 + 3);
        const int kb = 64 * s.sl, ke = 64 * (min(s.sh, jh) + 1);
        const int64_t r0 = (int64_t)I * 64;
        Acc acc;
        acc_zero(acc);
        block_gemm<1, 4, RowK, RowK>(E + r0 * ldw, ldw, 64, PA + (int64_t)j0 * 64 * lda, lda,
                                     64 * (jh - j0 + 1), kb, ke, lds, acc);
        block_store<1, 4>(Y + r0 * ldw + (int64_t)j0 * 64, ldw, 64, 64 * (jh - j0 + 1), 1.f, I < acc_rows ? 1.f : 0.f,
                          acc);
    }
}
// One stage-1 list entry's geometry: tile row I, target columns j0 .. jh,
// K range [kb, ke); false when the entry has no work.
struct RowEntry {
    int I, j0, jh, kb, ke;
    __device__ __forceinline__ bool load(const uint32_t* __restrict__ list, unsigned q, unsigned count, int K0,
                                         int mid, int y0, int y1, int Mt, int Nt)
    {
        if (q >= count) return false;
        const uint32_t e = list[xcd_entry(q, count)];
        I = (int)(e >> 16);
        const int b = (int)(e & 0xffffu);
        if (I < rows_lo(K0, Nt) || I > rows_hi(mid, Mt)) return false;
        const RowSpan s(I, K0, mid, y0, y1, Nt);
        j0 = s.tl + 4 * b;
        if (j0 > s.th) return false;
        jh = min(s.th, j0 + 3);
        kb = 64 * s.sl;
        ke = 64 * (min(s.sh, jh) + 1);
        return true;
    }
};

// A far part's stage 1 (the far twin of k_prop_rows, same blocks and
// results) on workgroups of 512 threads: the two 4-wave halves
// take list entries 2 p and 2 p + 1 of pair p = blockIdx.x, + gridDim.x, ...
// (neighbours in the longest-first list, so their K extents are close) and
// share each chunk barrier (dual_block_gemm).  Two 80 KB halves fill a CU's
// LDS, so no leaf runs beside one, and a CU keeps two blocks in flight.
__global__ __launch_bounds__(512) void k_prop_rows_far(const float* __restrict__ E, const float* __restrict__ PA,
                                                        float* __restrict__ Y, int64_t ldw, int64_t lda,
                                                        int K0, int mid, int y0, int y1, int Mt, int Nt,
                                                        const uint32_t* __restrict__ list, unsigned count,
                                                        int acc_rows)
{
    __shared__ __align__(16) float lds[2 * RowBlk::LDS_FLOATS];
    const int h = threadIdx.x >> 8;
    for (unsigned pr = blockIdx.x; 2 * pr < count; pr += gridDim.x) {
        int nother;
        {
            RowEntry o;
            nother = o.load(list, 2 * pr + (1 - h), count, K0, mid, y0, y1, Mt, Nt) ? (o.ke - o.kb) / kBK : 0;
        }
        RowEntry c;
        const bool ok = c.load(list, 2 * pr + h, count, K0, mid, y0, y1, Mt, Nt);
        const int nmax = max(ok ? (c.ke - c.kb) / kBK : 0, nother);
        const int64_t r0 = (int64_t)(ok ? c.I : 0) * 64, cc = (int64_t)(ok ? c.j0 : 0) * 64;
        const int cols = ok ? 64 * (c.jh - c.j0 + 1) : 64;
        Acc acc;
        acc_zero(acc);
        dual_block_gemm<1, 4, RowK, RowK>(E + r0 * ldw, ldw, 64, PA + cc * lda, lda, cols, ok ? c.kb : 0,
                                          ok ? c.ke : 0, nmax, lds + h * RowBlk::LDS_FLOATS, acc);
        if (ok) block_store<1, 4>(Y + r0 * ldw + cc, ldw, 64, cols, 1.f, c.I < acc_rows ? 1.f : 0.f, acc);
    }
}

__global__ __launch_bounds__(256, 2) void k_prop_rows(const float* __restrict__ E, const float* __restrict__ PA,
                                                   float* __restrict__ Y, int64_t ldw, int64_t lda,
                                                   int K0, int mid, int y0, int y1, int Mt, int Nt,
                                                   const uint32_t* __restrict__ list, unsigned count, int acc_rows)
{
    near_priority();
    prop_rows_body(E, PA, Y, ldw, lda, K0, mid, y0, y1, Mt, Nt, list, count, acc_rows);
}

// Stage 2 of node (K0, mid, K1), one part: block (column J, b) from the
// schedule updates the (up to) four target tile rows I' = i0 .. ih on the
// part's target anti-diagonals [t0, t1):
//   Wt[I', J] -= sum_{I = slo .. min(I', mid - 1)} P_B[I', I] Y[I, J],
// slo = max(0, K0 - J).
__device__ __forceinline__ void prop_cols_body(const float* __restrict__ Y, const float* __restrict__ PB,
                                               float* __restrict__ Wt, int64_t ldw, int64_t ldb,
                                               int K0, int mid, int t0, int t1, int Mt, int Nt,
                                               const uint32_t* __restrict__ list, unsigned count)
{
    __shared__ __align__(16) float lds[ColBlk::LDS_FLOATS];
    for (unsigned q = blockIdx.x; q < count; q += gridDim.x) {
        const uint32_t e = list[xcd_entry(q, count)];
        const int J = (int)(e >> 16), b = (int)(e & 0xffffu);
        if (J < cols_lo(t0, Mt) || J > cols_hi(t1, Nt)) continue;
        const ColSpan s(J, K0, mid, t0, t1, Mt);
        const int i0 = s.tl + 4 * b;
        if (i0 > s.th) continue;
        const int ih = min(s.th, i0 + 3);
        const int kb = 64 * s.slo, ke = 64 * (min(mid - 1, ih) + 1);
        const int64_t c0 = (int64_t)J * 64, rr = (int64_t)i0 * 64;
        Acc acc;
        acc_zero(acc);
        block_gemm<4, 1, RowK, KRow>(PB + rr * ldb, ldb, 64 * (ih - i0 + 1), Y + c0, ldw, 64, kb, ke, lds, acc);
        block_store<4, 1>(Wt + rr * ldw + c0, ldw, 64 * (ih - i0 + 1), 64, -1.f, 1.f, acc);
    }
}
__global__ __launch_bounds__(256, 2) void k_prop_cols(const float* __restrict__ Y, const float* __restrict__ PB,
                                                      float* __restrict__ Wt, int64_t ldw, int64_t ldb,
                                                      int K0, int mid, int t0, int t1, int Mt, int Nt,
                                                      const uint32_t* __restrict__ list, unsigned count)
{
    near_priority();
    prop_cols_body(Y, PB, Wt, ldw, ldb, K0, mid, t0, t1, Mt, Nt, list, count);
}
__global__ __launch_bounds__(256, 2) void k_prop_cols_far(const float* __restrict__ Y, const float* __restrict__ PB,
                                                          float* __restrict__ Wt, int64_t ldw, int64_t ldb,
                                                          int K0, int mid, int t0, int t1, int Mt, int Nt,
                                                          const uint32_t* __restrict__ list, unsigned count)
{
    prop_cols_body(Y, PB, Wt, ldw, ldb, K0, mid, t0, t1, Mt, Nt, list, count);
}

// Small parts: the same two stages with one 64 x 64 target tile per
// workgroup and one 32 x 32 quadrant per wave (block_gemm64), so a part with
// few 64 x 256 blocks still spreads over many CUs.
// Work item q = y * span + x (x fastest), taken by workgroups blockIdx.x,
// blockIdx.x + gridDim.x, ... as in the block kernels.
// Stage 1: item (x, y) computes Y[I, J'] for row I = rows_lo + y and
// J' = th - x (the K extent grows with J': longest first).
__device__ __forceinline__ void prop_rows_t_body(const float* __restrict__ E, const float* __restrict__ PA,
                                                 float* __restrict__ Y, int64_t ldw, int64_t lda,
                                                 int K0, int mid, int y0, int y1, int Nt, unsigned span,
                                                 unsigned count, int acc_rows)
{
    __shared__ __align__(16) float lds[kLds64];
    const int wave = threadIdx.x >> 6;
    for (unsigned qq = blockIdx.x; qq < count; qq += gridDim.x) {
        const unsigned q = kTileXcd ? xcd_entry(qq, count) : qq;
        const int I = rows_lo(K0, Nt) + (int)(q / span);
        const RowSpan s(I, K0, mid, y0, y1, Nt);
        const int Jp = s.th - (int)(q % span);
        if (Jp < s.tl) continue;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        block_gemm64<RowK, RowK>(E + (int64_t)I * 64 * ldw, ldw, PA + (int64_t)Jp * 64 * lda, lda, 64 * s.sl,
                                 64 * (min(s.sh, Jp) + 1), lds, acc);
        const int64_t r = (int64_t)I * 64 + 32 * (wave >> 1);
        const int64_t c = (int64_t)Jp * 64 + 32 * (wave & 1);
        wave_store32(Y + r * ldw + c, ldw, 1.f, I < acc_rows ? 1.f : 0.f, acc);
    }
}
__global__ __launch_bounds__(256) void k_prop_rows_t(const float* __restrict__ E, const float* __restrict__ PA,
                                                     float* __restrict__ Y, int64_t ldw, int64_t lda,
                                                     int K0, int mid, int y0, int y1, int Nt, unsigned span,
                                                     unsigned count, int acc_rows)
{
    near_priority();
    prop_rows_t_body(E, PA, Y, ldw, lda, K0, mid, y0, y1, Nt, span, count, acc_rows);
}
__global__ __launch_bounds__(256) void k_prop_rows_t_far(const float* __restrict__ E, const float* __restrict__ PA,
                                                         float* __restrict__ Y, int64_t ldw, int64_t lda,
                                                         int K0, int mid, int y0, int y1, int Nt, unsigned span,
                                                         unsigned count, int acc_rows)
{
    prop_rows_t_body(E, PA, Y, ldw, lda, K0, mid, y0, y1, Nt, span, count, acc_rows);
}

// Stage 2: item (x, y) updates Wt[I', J] for column J = cols_lo + y and
// I' = th - x.
__device__ __forceinline__ void prop_cols_t_body(const float* __restrict__ Y, const float* __restrict__ PB,
                                                 float* __restrict__ Wt, int64_t ldw, int64_t ldb,
                                                 int K0, int mid, int t0, int t1, int Mt, unsigned span,
                                                 unsigned count)
{
    __shared__ __align__(16) float lds[kLds64];
    const int wave = threadIdx.x >> 6;
    for (unsigned qq = blockIdx.x; qq < count; qq += gridDim.x) {
        const unsigned q = kTileXcd ? xcd_entry(qq, count) : qq;
        const int J = cols_lo(t0, Mt) + (int)(q / span);
        const ColSpan s(J, K0, mid, t0, t1, Mt);
        const int Ip = s.th - (int)(q % span);
        if (Ip < s.tl) continue;
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        block_gemm64<RowK, KRow>(PB + (int64_t)Ip * 64 * ldb, ldb, Y + (int64_t)J * 64, ldw, 64 * s.slo,
                                 64 * (min(mid - 1, Ip) + 1), lds, acc);
        const int64_t r = (int64_t)Ip * 64 + 32 * (wave >> 1);
        const int64_t c = (int64_t)J * 64 + 32 * (wave & 1);
        wave_store32(Wt + r * ldw + c, ldw, -1.f, 1.f, acc);
    }
}
__global__ __launch_bounds__(256) void k_prop_cols_t(const float* __restrict__ Y, const float* __restrict__ PB,
                                                     float* __restrict__ Wt, int64_t ldw, int64_t ldb,
                                                     int K0, int mid, int t0, int t1, int Mt, unsigned span,
                                                     unsigned count)
{
    near_priority();
    prop_cols_t_body(Y, PB, Wt, ldw, ldb, K0, mid, t0, t1, Mt, span, count);
}
__global__ __launch_bounds__(256) void k_prop_cols_t_far(const float* __restrict__ Y, const float* __restrict__ PB,
                                                         float* __restrict__ Wt, int64_t ldw, int64_t ldb,
                                                         int K0, int mid, int t0, int t1, int Mt, unsigned span,
                                                         unsigned count)
{
    prop_cols_t_body(Y, PB, Wt, ldw, ldb, K0, mid, t0, t1, Mt, span, count);
}

__global__ __launch_bounds__(256) void k_obj_reduce(const double* __restrict__ part, int64_t count,
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

struct SolvePlan {
    int64_t m, n, Mt, Nt, Mp, Np;
    bool pad_a, pad_b;
    SchedGeom sg;
    int64_t sched_entries;
    int split_levels;   // depths 0 .. split_levels - 1 may hold split nodes
    size_t off_wt, off_e, off_y, off_obj, off_pa, off_pb, off_sched, total;
    size_t off_ysplit[kSplitDepth];   // one stage-1 buffer per depth with split nodes
};

// Heap levels holding internal nodes, and the list offsets of k_sched.
void plan_sched(SchedGeom& g, int64_t& entries, int Mt, int Nt)
{
    g.Mt = Mt;
    g.Nt = Nt;
    g.Kt = Mt + Nt - 1;
    g.levels = 0;
    while ((1 << g.levels) < g.Kt) ++g.levels;   // depth d holds a node of width >= 2 iff 2^d < Kt
    // the widest node at depth d is ceil(Kt / 2^d) wide, its right child
    // half of that (rounded up)
    g.split_depth = 0;
    while (g.split_depth < std::min(kSplitDepth, g.levels) &&
           ceil_div(ceil_div(g.Kt, (int64_t)1 << g.split_depth), 2) >= kSplitMin)
        ++g.split_depth;
    g.split3_depth = std::min(kSplit3Depth, g.split_depth);
    g.early_depth = std::min(kEarlyDepth, g.split_depth);
    const int64_t R = std::max(Mt, Nt);
    int64_t off = 0;
    for (int d = 0; d < kMaxDepth; ++d) {
        const int64_t w = ceil_div(g.Kt, (int64_t)1 << d);
        g.base[d] = off;
        g.cap[d] = R * ceil_div(w, 4);
        if (d < g.levels) off += ((int64_t)1 << d) * kNodeLists * g.cap[d];   // 2 stages x kMaxParts parts + the early pass
    }
    entries = off;
}

SolvePlan plan_solve(int64_t m, int64_t n, bool split)
{
    SolvePlan p;
    p.m = m;
    p.n = n;
    p.Mt = ceil_div(m, kTile);
    p.Nt = ceil_div(n, kTile);
    p.Mp = p.Mt * kTile;
    p.Np = p.Nt * kTile;
    p.pad_a = (n % kTile) != 0;
    p.pad_b = (m % kTile) != 0;
    plan_sched(p.sg, p.sched_entries, (int)p.Mt, (int)p.Nt);
    if (!split) p.sg.split_depth = p.sg.split3_depth = 0;
    p.split_levels = p.sg.split_depth;
    const size_t mat = sizeof(float) * (size_t)(p.Mp * p.Np);
    size_t off = 0;
    p.off_wt = off;
    off = align_up(off + mat);
    p.off_e = off;
    off = align_up(off + mat);
    p.off_y = off;
    off = align_up(off + mat);
    for (int d = 0; d < kSplitDepth; ++d) {
        p.off_ysplit[d] = off;
        if (d < p.split_levels) off = align_up(off + mat);
    }
    p.off_obj = off;
    off = align_up(off + sizeof(double) * (size_t)(p.Mt * p.Nt));
    p.off_pa = p.off_pb = 0;
    if (p.pad_a) {
        p.off_pa = off;
        off = align_up(off + sizeof(float) * (size_t)(p.Np * p.Np));
    }
    if (p.pad_b) {
        p.off_pb = off;
        off = align_up(off + sizeof(float) * (size_t)(p.Mp * p.Mp));
    }
    p.off_sched = off;
    off = align_up(off + sizeof(uint32_t) * (size_t)p.sched_entries);
    p.total = off;
    return p;
}

dim3 copy_grid(int64_t R, int64_t C)
{
    return dim3((unsigned)ceil_div(C, 1024), (unsigned)std::min<int64_t>(R, 32768));
}

int copy_vec(const float* src, int64_t lds) { return (lds % 4 == 0 && aligned16(src)) ? 1 : 0; }

struct SolveRun {
    LeafArgs leaf;
    float* Y;                      // stage-1 buffer of unsplit nodes
    float* Ysplit[kSplitDepth];    // ... of the split nodes at each depth
    const uint32_t* sched;
    const SchedGeom* sg;
    int Mt, Nt;
    hipStream_t s;                 // the caller's stream: leaves, unsplit nodes, near parts
    hipStream_t far[kSplitDepth];  // far parts of split nodes, one stream per depth
    std::vector<hipEvent_t> events;
    bool failed;
    Prof* prof;
    // Factors still being computed (SolveWait), per factor f: event k of
    // ev[f] makes tile rows / columns below Kq[f][k] final (the last one,
    // the whole factor, has Kq = INT_MAX); waited[f] is the last one waited for.
    int nwait[2] = {0, 0};
    int Kq[2][kMaxLeads + 1];
    hipEvent_t ev[2][kMaxLeads + 1];
    int waited[2] = {-1, -1};
};

// Before work that reads the factors on tile anti-diagonals up to khi (so
// on tile rows and columns up to khi): wait for the first event of each
// factor whose block reaches beyond khi, unless a later one was waited for.
// Each factor's events complete in order (one stream), so one wait covers
// the earlier ones.
void ensure_full(SolveRun& R, int khi)
{
    for (int f = 0; f < 2; ++f) {
        int k = 0;
        while (k < R.nwait[f] && R.Kq[f][k] <= khi) ++k;
        if (k >= R.nwait[f] || k <= R.waited[f]) continue;
        R.waited[f] = k;
        if (hipStreamWaitEvent(R.s, R.ev[f][k], 0) != hipSuccess) R.failed = true;
    }
}

// The same for work on another stream (an early source pass): that stream
// waits; the caller's stream is not affected.
void ensure_full_on(SolveRun& R, hipStream_t st, int khi)
{
    for (int f = 0; f < 2; ++f) {
        int k = 0;
        while (k < R.nwait[f] && R.Kq[f][k] <= khi) ++k;
        if (k < R.nwait[f] && hipStreamWaitEvent(st, R.ev[f][k], 0) != hipSuccess) R.failed = true;
    }
}

hipEvent_t new_event(SolveRun& R)
{
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
        R.failed = true;
        return nullptr;
    }
    R.events.push_back(e);
    return e;
}

int launch_ok() { return hipGetLastError() == hipSuccess ? 0 : -1; }

constexpr double kTileB = 4.0 * 64 * 64;                 // bytes of one fp32 tile
constexpr double kFull = 64.0 * 64.0 * 64.0;             // multiply-adds of a full block product
constexpr double kTriB = 64.0 * 64.0 * 65.0 / 2.0;       // ... with a triangular diagonal block

// nsrc > 0: K is the (nsrc + 1)-th leaf of a narrow node, and the leaf
// applies the errors of the node's earlier leaves first.
void enqueue_leaf(SolveRun& R, int K, int nsrc = 0)
{
    const int I_lo = std::max(0, K - (R.Nt - 1));
    const int I_hi = std::min(R.Mt - 1, K);
    const int count = I_hi - I_lo + 1;
    R.leaf.K = K;
    R.leaf.I_lo = I_lo;
    R.leaf.nsrc = nsrc;
    // per tile: the two in-tile triangular products (U = E P_A^T, P_B U);
    // bytes: W~, P_A and P_B diagonal blocks in; E and V out (+ err), codes.
    // (A leaf that first applies its narrow node's propagation does that
    // node's block products too, on the MFMA units; they are not counted
    // here, so the leaf's rate is that of its sweep.)
    const double flops = count * 2.0 * 2.0 * kTriB;
    const double bytes = count * (5.0 * kTileB + (R.leaf.err ? kTileB : 0.0) + 64.0 * 64.0);
    launch(R.prof, KK_LEAF, flops, bytes, k_leaf, dim3(count), dim3(512), R.s, R.leaf);
}

// A stage with fewer 64 x 256 blocks than this runs one 64 x 64 tile per
// workgroup instead (k_prop_rows_t / k_prop_cols_t).
#ifndef BAKRON_BLOCK_LAUNCH_MIN
#define BAKRON_BLOCK_LAUNCH_MIN 512
#endif
constexpr int64_t kBlockLaunchMin = BAKRON_BLOCK_LAUNCH_MIN;

// A far part runs beside the leaves and small nodes of the caller's stream,
// which are latency-bound: a leaf sharing a CU with a propagation workgroup
// runs about three times slower.  So a far launch takes at most kFarGrid
// workgroups (looping over its blocks) and reserves enough extra LDS that no
// leaf fits next to one of them: leaves then run on CUs of their own.  (The
// far stage-1 block kernel needs no reserve: its 512-thread workgroups work
// on two blocks at once and fill a CU's LDS by themselves.)
#ifndef BAKRON_FAR_GRID
#define BAKRON_FAR_GRID 192
#endif
constexpr unsigned kFarGrid = BAKRON_FAR_GRID;
// Far parts switch to the block kernels much earlier than near ones: on the
// capped grid each workgroup has a CU to itself (the LDS reserve), where a
// 64 x 64 tile keeps one MFMA accumulator chain per SIMD busy and a 64 x 256
// block four.
#ifndef BAKRON_FAR_BLOCK_MIN
#define BAKRON_FAR_BLOCK_MIN 128
#endif
constexpr int64_t kFarBlockMin = BAKRON_FAR_BLOCK_MIN;   // the block kernel from this many blocks
constexpr size_t kLdsPerCU = 160 * 1024;
constexpr size_t kLeafLds = sizeof(float) * (64 * 64 + 3 * 64 * kLP + 8) + 64 * 64 + 8 * sizeof(double);   // k_leaf's arrays
static_assert(kLeafLds == kLeafLdsBytes, "k_leaf's LDS as the factor's lead launches assume it");
constexpr size_t pad_to_exclude(size_t static_lds)
{
    return static_lds + kLeafLds > kLdsPerCU ? 0 : kLdsPerCU - kLeafLds - static_lds + 1024;
}
constexpr size_t kFarPadBlock = pad_to_exclude(sizeof(float) * RowBlk::LDS_FLOATS);
#ifndef BAKRON_FAR_PAD_TILE
#define BAKRON_FAR_PAD_TILE 1
#endif
constexpr size_t kFarPadTile = BAKRON_FAR_PAD_TILE ? pad_to_exclude(sizeof(float) * kLds64) : 0;
static_assert(sizeof(float) * RowBlk::LDS_FLOATS == sizeof(float) * ColBlk::LDS_FLOATS, "one pad for both stages");

// Stage 1 of one part of node (K0, mid, K1) on stream st into Y (sources
// [K0, mid); rows I < acc_rows add to Y).
void enqueue_stage1(SolveRun& R, int K0, int mid, int y0, int y1, const uint32_t* list, float* Y, hipStream_t st,
                    bool far, int acc_rows, unsigned grid_cap = kFarGrid)
{
    const int Mt = R.Mt, Nt = R.Nt;
    const int I_lo = rows_lo(K0, Nt), I_hi = rows_hi(mid, Mt);
    int64_t blocks = 0;
    int span = 0;   // widest row, in target tiles
    double fl = 0.0, by = 0.0;
    std::vector<uint8_t> pa_used;
    if (R.prof) pa_used.assign((size_t)Nt * Nt, 0);
    for (int I = I_lo; I <= I_hi; ++I) {
        const RowSpan sp(I, K0, mid, y0, y1, Nt);
        blocks += sp.blocks();
        span = std::max(span, sp.th - sp.tl + 1);
        if (R.prof && sp.th >= sp.tl) {
            // pairs (J, J') with sl <= J <= min(sh, J'); the diagonal block is triangular
            for (int Jp = sp.tl; Jp <= sp.th; ++Jp) {
                const int hi = std::min(sp.sh, Jp);
                const double cnt = hi - sp.sl + 1;
                const bool diag = Jp <= sp.sh;
                fl += 2.0 * ((cnt - (diag ? 1 : 0)) * kFull + (diag ? kTriB : 0.0));
                for (int J = sp.sl; J <= hi; ++J) pa_used[(size_t)Jp * Nt + J] = 1;
            }
            by += ((sp.sh - sp.sl + 1) + (sp.th - sp.tl + 1)) * kTileB;   // E read, Y written
        }
    }
    if (R.prof)   // distinct P_A blocks
        for (uint8_t u : pa_used) by += u ? kTileB : 0.0;
    if (far && blocks >= kFarBlockMin) {
        const unsigned n = (unsigned)blocks;
        launch(R.prof, KK_PROP_ROWS_FAR, fl, by, k_prop_rows_far, dim3(std::min((n + 1) / 2, grid_cap)), dim3(512),
               st, (const float*)R.leaf.E, R.leaf.PA, Y, R.leaf.ldw, R.leaf.lda, K0, mid, y0, y1, Mt, Nt, list, n,
               acc_rows);
    } else if (blocks >= kBlockLaunchMin) {
        const unsigned n = (unsigned)blocks;
        launch(R.prof, KK_PROP_ROWS, fl, by, k_prop_rows, dim3(n), dim3(256), st, (const float*)R.leaf.E, R.leaf.PA,
               Y, R.leaf.ldw, R.leaf.lda, K0, mid, y0, y1, Mt, Nt, list, n, acc_rows);
    } else if (blocks > 0) {
        const unsigned n = (unsigned)span * (unsigned)(I_hi - I_lo + 1);
        launch_shm(R.prof, far ? KK_PROP_ROWS_T_FAR : KK_PROP_ROWS_T, fl, by, far ? k_prop_rows_t_far : k_prop_rows_t, dim3(far ? std::min(n, grid_cap) : n), dim3(256),
                   far ? kFarPadTile : 0, st, (const float*)R.leaf.E, R.leaf.PA, Y, R.leaf.ldw, R.leaf.lda, K0, mid,
                   y0, y1, Nt, (unsigned)span, n, acc_rows);
    }
}

// Stage 2 of one part of node (K0, mid, K1) (targets [t0, t1)) on stream st from Y.
void enqueue_stage2(SolveRun& R, int K0, int mid, int t0, int t1, const uint32_t* list, const float* Y,
                    hipStream_t st, bool far)
{
    const int Mt = R.Mt, Nt = R.Nt;
    const int J_lo = cols_lo(t0, Mt), J_hi = cols_hi(t1, Nt);
    int64_t blocks = 0;
    int span = 0;
    double fl = 0.0, by = 0.0;
    std::vector<uint8_t> pb_used;
    if (R.prof) pb_used.assign((size_t)Mt * Mt, 0);
    for (int J = J_lo; J <= J_hi; ++J) {
        const ColSpan sp(J, K0, mid, t0, t1, Mt);
        blocks += sp.blocks();
        span = std::max(span, sp.th - sp.tl + 1);
        if (R.prof && sp.th >= sp.tl) {
            for (int Ip = sp.tl; Ip <= sp.th; ++Ip) {
                const int shi = std::min(mid - 1, Ip);
                const double cnt = shi - sp.slo + 1;
                const bool diag = Ip <= mid - 1;
                fl += 2.0 * ((cnt - (diag ? 1 : 0)) * kFull + (diag ? kTriB : 0.0));
                for (int I = sp.slo; I <= shi; ++I) pb_used[(size_t)Ip * Mt + I] = 1;
            }
            by += (std::min(mid - 1, sp.th) - sp.slo + 1) * kTileB;   // Y read
            by += 2.0 * (sp.th - sp.tl + 1) * kTileB;                 // W~ read and written
        }
    }
    if (R.prof)   // distinct P_B blocks
        for (uint8_t u : pb_used) by += u ? kTileB : 0.0;
    if (blocks >= (far ? kFarBlockMin : kBlockLaunchMin)) {
        const unsigned n = (unsigned)blocks;
        launch_shm(R.prof, far ? KK_PROP_COLS_FAR : KK_PROP_COLS, fl, by, far ? k_prop_cols_far : k_prop_cols, dim3(far ? std::min(n, kFarGrid) : n), dim3(256),
                   far ? kFarPadBlock : 0, st, Y, R.leaf.PB, R.leaf.Wt, R.leaf.ldw, R.leaf.ldb, K0, mid, t0, t1, Mt,
                   Nt, list, n);
    } else if (blocks > 0) {
        const unsigned n = (unsigned)span * (unsigned)(J_hi - J_lo + 1);
        launch_shm(R.prof, far ? KK_PROP_COLS_T_FAR : KK_PROP_COLS_T, fl, by, far ? k_prop_cols_t_far : k_prop_cols_t, dim3(far ? std::min(n, kFarGrid) : n), dim3(256),
                   far ? kFarPadTile : 0, st, Y, R.leaf.PB, R.leaf.Wt, R.leaf.ldw, R.leaf.ldb, K0, mid, t0, t1, Mt,
                   (unsigned)span, n);
    }
}

// Events due before the propagation of the nodes down a left spine:
// e[j] for the node j levels below (e[0]: the node itself).
struct SpineWaits {
    hipEvent_t e[kMaxParts];
};

// An early source pass (the node's stage 1 over the sources [K0, q), every
// Y column) on stream fs, once the caller's stream has solved [K0, q) and
// enqueued the left child's propagation; `done` is recorded after it.
struct EarlyPass {
    int K0, mid, K1, d, p;
    hipEvent_t done;
};

void enqueue_early(SolveRun& R, EarlyPass& e, hipStream_t fs)
{
    const SchedGeom& g = *R.sg;
    hipEvent_t ready = new_event(R);   // the errors of [K0, q) are final
    if (!ready || hipEventRecord(ready, R.s) != hipSuccess || hipStreamWaitEvent(fs, ready, 0) != hipSuccess) {
        R.failed = true;
        return;
    }
    ensure_full_on(R, fs, e.K1 - 1);   // P_A rows up to K1 - 1
    const uint32_t* list = R.sched + g.base[e.d] + (int64_t)(kNodeLists * e.p + 2 * kMaxParts) * g.cap[e.d];
    enqueue_stage1(R, e.K0, (e.K0 + e.mid) / 2, e.K0, e.K1, list, R.Ysplit[e.d], fs, true, 0, kEarlyGrid);
    e.done = new_event(R);
    if (!e.done || hipEventRecord(e.done, fs) != hipSuccess) R.failed = true;
}

// Node (K0, mid, K1) at heap position (d, p).  Unsplit: both stages on the
// caller's stream.  Cut in parts: the first part on the caller's stream,
// the others in order on the depth's own stream once the first part's
// stage 1 is done (later parts read its Y columns too).  Part k >= 1 ends
// with an event, due before the propagation of the node parts - 1 - k
// levels down the left spine of the right child (the first work on the
// caller's stream that touches the part's targets): returned in `done`.
// An early node's stage 1 takes the late sources [q, mid) on top of its
// early pass: that pass ran on the depth's stream (early_done, waited for
// here) or, when the node is not split, runs here first.
void enqueue_prop(SolveRun& R, int K0, int mid, int K1, int d, int p, SpineWaits& done, hipEvent_t early_done)
{
    for (hipEvent_t& e : done.e) e = nullptr;
    const SchedGeom& g = *R.sg;
    const uint32_t* lists = R.sched + g.base[d] + (int64_t)(kNodeLists * p) * g.cap[d];   // (stage, part) at (kMaxParts stage + part) cap
    const int parts = node_parts(g, d, mid, K1);
    float* Y = parts > 1 ? R.Ysplit[d] : R.Y;
    const bool early = node_early(g, d, K0, mid, K1);
    const int q = (K0 + mid) / 2;
    const int sk0 = early ? q : K0, acc_rows = early ? q : 0;   // the stage-1 sources of the parts: [sk0, mid)
    if (early) {
        if (early_done) {
            if (hipStreamWaitEvent(R.s, early_done, 0) != hipSuccess) R.failed = true;
        } else {
            enqueue_stage1(R, K0, q, K0, K1, lists + 2 * kMaxParts * g.cap[d], Y, R.s, false, 0);
        }
    }
    const PartRange p0(parts, 0, K0, mid, K1);
    enqueue_stage1(R, sk0, mid, p0.y0, p0.y1, lists, Y, R.s, false, acc_rows);
    if (parts == 1) {
        enqueue_stage2(R, K0, mid, p0.t0, p0.t1, lists + kMaxParts * g.cap[d], Y, R.s, false);
        return;
    }
    hipEvent_t ev0 = new_event(R);
    if (!ev0) return;
    if (hipEventRecord(ev0, R.s) != hipSuccess || hipStreamWaitEvent(R.far[d], ev0, 0) != hipSuccess) {
        R.failed = true;
        return;
    }
    enqueue_stage2(R, K0, mid, p0.t0, p0.t1, lists + kMaxParts * g.cap[d], Y, R.s, false);
    for (int part = 1; part < parts; ++part) {
        const PartRange pr(parts, part, K0, mid, K1);
        enqueue_stage1(R, sk0, mid, pr.y0, pr.y1, lists + part * g.cap[d], Y, R.far[d], true, acc_rows);
        enqueue_stage2(R, K0, mid, pr.t0, pr.t1, lists + (kMaxParts + part) * g.cap[d], Y, R.far[d], true);
        hipEvent_t ev = new_event(R);
        if (!ev || hipEventRecord(ev, R.far[d]) != hipSuccess) {
            R.failed = true;
            return;
        }
        done.e[parts - 1 - part] = ev;
    }
}

// `waits`: far parts of ancestors due before the propagation of this node
// and of the nodes down its left spine.  `parent`: the early pass of the
// parent node when this is its left child.  It is enqueued after this
// node's propagation, behind this node's far parts on their stream (or on
// the parent's stream when this node is not split): the caller's stream
// then runs the leaves of this node's right child, and the early pass takes
// CUs beside them rather than beside this node's near part or its far
// parts.  A node of at most kFold anti-diagonals has no propagation
// launches: each of its leaves applies the errors of the node's earlier
// leaves first (leaf_prologue), and the waits come before the leaves at the
// recursion's propagation points.
// (Three or four anti-diagonals: each leaf's prologue then does up to 13
// block products on its one CU, which costs more than the two tile
// launches it saves.)
#ifndef BAKRON_FOLD
#define BAKRON_FOLD 2
#endif
constexpr int kFold = BAKRON_FOLD;
void solve_rec(SolveRun& R, int K0, int K1, int d, int p, const SpineWaits& waits, EarlyPass* parent)
{
    if (K1 - K0 == 1) {   // (the nodes that carry waits or an early pass are never leaves)
        ensure_full(R, K0);
        enqueue_leaf(R, K0);
        return;
    }
    if (K1 - K0 <= kFold) {   // (never split, never an early node)
        int mids[kMaxParts];   // propagation point of the node j levels down the left spine
        for (int j = 0, hi = K1; j < kMaxParts; ++j) {
            mids[j] = hi - K0 >= 2 ? (K0 + hi) / 2 : -1;
            hi = mids[j] < 0 ? hi : mids[j];
        }
        for (int K = K0; K < K1; ++K) {
            for (int j = kMaxParts - 1; j >= 0; --j)
                if (waits.e[j] && K == mids[j] && hipStreamWaitEvent(R.s, waits.e[j], 0) != hipSuccess) R.failed = true;
            ensure_full(R, K);
            enqueue_leaf(R, K, K - K0);
        }
        return;
    }
    const int mid = (K0 + K1) / 2;
    SpineWaits down;
    for (int j = 0; j < kMaxParts; ++j) down.e[j] = j + 1 < kMaxParts ? waits.e[j + 1] : nullptr;
    // a split early node runs its early pass on its depth's stream
    EarlyPass mine{K0, mid, K1, d, p, nullptr};
    const bool early_far = node_early(*R.sg, d, K0, mid, K1) && node_parts(*R.sg, d, mid, K1) > 1;
    solve_rec(R, K0, mid, d + 1, 2 * p, down, early_far ? &mine : nullptr);
    if (waits.e[0] && hipStreamWaitEvent(R.s, waits.e[0], 0) != hipSuccess) R.failed = true;
    ensure_full(R, K1 - 1);
    SpineWaits done;
    enqueue_prop(R, K0, mid, K1, d, p, done, mine.done);
    if (parent) enqueue_early(R, *parent, node_parts(*R.sg, d, mid, K1) > 1 ? R.far[d] : R.far[parent->d]);
    solve_rec(R, mid, K1, d + 1, 2 * p + 1, done, nullptr);
}

}  // namespace

size_t solve_workspace_bytes(int64_t m, int64_t n, bool split)
{
    if (m <= 0 || n <= 0) return 0;
    return plan_solve(m, n, split).total;
}

int solve_enqueue(const float* W, int64_t m, int64_t n, const float* LA, const float* PA,
                  const float* LB, const float* PB, const float* scale, const float* zero,
                  const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                  void* ws, hipStream_t s, Prof* prof, bool split, const SolveWait* wait, int64_t group_size)
{
    SolvePlan p = plan_solve(m, n, split);
    char* w = static_cast<char*>(ws);
    SolveRun R;
    R.prof = prof;
    R.s = s;
    R.failed = false;
    if (wait) {
        // The padded copies of P_A and P_B need the whole factors.
        const bool whole = p.pad_a || p.pad_b;
        for (int f = 0; f < 2; ++f) {
            int k = 0;
            for (int j = 0; !whole && j < wait->lead[f].count; ++j) {
                R.Kq[f][k] = (int)(wait->lead[f].size[j] / kTile);
                R.ev[f][k++] = wait->lead[f].ev[j];
            }
            R.Kq[f][k] = INT_MAX;
            R.ev[f][k++] = wait->full[f];
            R.nwait[f] = k;
        }
        if (whole) ensure_full(R, 0);
    }
    for (int d = 0; d < kSplitDepth; ++d) {
        R.Ysplit[d] = d < p.sg.split_depth ? reinterpret_cast<float*>(w + p.off_ysplit[d]) : nullptr;
        R.far[d] = d < p.sg.split_depth ? side_stream(d) : nullptr;
        if (d < p.sg.split_depth && !R.far[d]) p.sg.split_depth = p.sg.split3_depth = 0;   // no stream: nothing is split
    }
    LeafArgs& g = R.leaf;
    g.Wt = reinterpret_cast<float*>(w + p.off_wt);
    g.E = reinterpret_cast<float*>(w + p.off_e);
    g.ldw = p.Np;
    R.Y = reinterpret_cast<float*>(w + p.off_y);
    const double dm = (double)m, dn = (double)n;
    if (p.pad_a) {
        float* pa = reinterpret_cast<float*>(w + p.off_pa);
        launch(prof, KK_COPY_PAD, 0.0, 4.0 * (dn * dn + (double)(p.Np * p.Np)), k_copy_pad, copy_grid(p.Np, p.Np),
               dim3(256), s, PA, n, n, n, pa, p.Np, p.Np, p.Np, copy_vec(PA, n));
        g.PA = pa;
        g.lda = p.Np;
    } else {
        g.PA = PA;
        g.lda = n;
    }
    if (p.pad_b) {
        float* pb = reinterpret_cast<float*>(w + p.off_pb);
        launch(prof, KK_COPY_PAD, 0.0, 4.0 * (dm * dm + (double)(p.Mp * p.Mp)), k_copy_pad, copy_grid(p.Mp, p.Mp),
               dim3(256), s, PB, m, m, m, pb, p.Mp, p.Mp, p.Mp, copy_vec(PB, m));
        g.PB = pb;
        g.ldb = p.Mp;
    } else {
        g.PB = PB;
        g.ldb = m;
    }
    launch(prof, KK_COPY_PAD, 0.0, 4.0 * (dm * dn + (double)(p.Mp * p.Np)), k_copy_pad, copy_grid(p.Mp, p.Np),
           dim3(256), s, W, m, n, n, g.Wt, p.Mp, p.Np, p.Np, copy_vec(W, n));
    if (launch_ok()) return -1;
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
    g.LB = LB;
    g.objp = objective ? reinterpret_cast<double*>(w + p.off_obj) : nullptr;
    g.Nt = (int)p.Nt;
    g.vec_out = (m % kTile == 0 && n % kTile == 0 && (reinterpret_cast<uintptr_t>(codes) & 15u) == 0 &&
                 aligned16(V) && (err == nullptr || aligned16(err)))
                    ? 1
                    : 0;
    R.Mt = (int)p.Mt;
    R.Nt = (int)p.Nt;
    R.sg = &p.sg;
    uint32_t* sched = reinterpret_cast<uint32_t*>(w + p.off_sched);
    R.sched = sched;
    if (p.sg.levels > 0)
        launch(prof, KK_SCHED, 0.0, 4.0 * (double)p.sched_entries, k_sched,
               dim3((unsigned)((1u << p.sg.levels) - 1u), 3u, (unsigned)kMaxParts), dim3(256), s, p.sg, sched);
    if (p.sg.split_depth > 0) {
        static std::once_flag attrs;
        std::call_once(attrs, [] {
            (void)hipFuncSetAttribute((const void*)k_prop_cols_far, hipFuncAttributeMaxDynamicSharedMemorySize,
                                      (int)kFarPadBlock);
            if (kFarPadTile) {
                (void)hipFuncSetAttribute((const void*)k_prop_rows_t_far, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)kFarPadTile);
                (void)hipFuncSetAttribute((const void*)k_prop_cols_t_far, hipFuncAttributeMaxDynamicSharedMemorySize,
                                          (int)kFarPadTile);
            }
        });
    }
    SpineWaits none;
    for (hipEvent_t& e : none.e) e = nullptr;
    solve_rec(R, 0, R.Mt + R.Nt - 1, 0, 0, none, nullptr);
    ensure_full(R, INT_MAX - 1);   // s is ordered after the factors in any case
    // every far part is waited for by the right child of its node, so all
    // of them are ordered before the rest of the work on s
    for (hipEvent_t e : R.events) (void)hipEventDestroy(e);
    if (R.failed || launch_ok()) return -1;
    if (objective) {
        const double cnt = (double)(p.Mt * p.Nt);
        launch(prof, KK_OBJ_REDUCE, cnt, 8.0 * (cnt + 1.0), k_obj_reduce, dim3(1), dim3(256), s,
               (const double*)g.objp, p.Mt * p.Nt, objective);
        if (launch_ok()) return -1;
    }
    return 0;
}

}  // namespace bk
