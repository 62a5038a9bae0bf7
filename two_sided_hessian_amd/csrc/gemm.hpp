// gemm.hpp -- fp32 MFMA block GEMM core for gfx950 (CDNA4).
//
// One workgroup = 4 waves (256 threads) computes a (64*WM) x (64*WN) output
// block; each wave owns one 64 x 64 sub-block as 2 x 2 tiles of
// v_mfma_f32_32x32x2f32 (32 x 32 output, K = 2 per instruction, 16 fp32
// accumulators per lane).  Operands are staged through LDS in K chunks of
// kBK, double-buffered, with the next chunk's global loads issued before the
// current chunk's MFMAs.  LDS holds both operands K-major ([k][row]) so the
// MFMA fragment reads are unit-stride across lanes.
//
// Every row/column extent used by the callers is a multiple of 64, so
// per-float4 bounds checks (rows beyond `rlim` read as zero) are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 16;   // K chunk staged in LDS
constexpr int kPad = 4;   // LDS row padding in floats (keeps 16-byte alignment)

// How an operand is stored in global memory, for operand element (r, k)
// where r runs over the output rows (operand A) or output columns (operand B):
//   RowK: p[r * ld + k]   (K contiguous)
//   KRow: p[k * ld + r]   (r contiguous)
enum Layout { RowK = 0, KRow = 1 };

template <int R>
struct OperandTile {
    static constexpr int LD = R + kPad;               // LDS row pitch (floats)
    static constexpr int F4 = R * kBK / 4;            // float4s per chunk
    static constexpr int PER_THREAD = F4 / 256;       // float4s per thread
    static_assert(F4 % 256 == 0, "tile too small for 256 threads");
};

// Global -> registers for one K chunk [k0, k0 + kBK) of an R-row operand.
template <int R, int LAYOUT>
__device__ __forceinline__ void load_chunk(const float* __restrict__ p, int64_t ld, int rlim,
                                           int k0, f32x4 (&reg)[OperandTile<R>::PER_THREAD])
{
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < OperandTile<R>::PER_THREAD; ++u) {
        const int f = t + 256 * u;
        int r, k;
        if (LAYOUT == KRow) {
            k = f / (R / 4);
            r = 4 * (f % (R / 4));
        } else {
            r = f / (kBK / 4);
            k = 4 * (f % (kBK / 4));
        }
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (r < rlim) {
            const float* src = (LAYOUT == KRow) ? p + (int64_t)(k0 + k) * ld + r
                                                : p + (int64_t)r * ld + (k0 + k);
            v = *reinterpret_cast<const f32x4*>(src);
        }
        reg[u] = v;
    }
}

// Registers -> LDS (K-major [k][r], pitch OperandTile<R>::LD).
template <int R, int LAYOUT>
__device__ __forceinline__ void store_chunk(float* __restrict__ s,
                                            const f32x4 (&reg)[OperandTile<R>::PER_THREAD])
{
    constexpr int LD = OperandTile<R>::LD;
    const int t = threadIdx.x;
#pragma unroll
    for (int u = 0; u < OperandTile<R>::PER_THREAD; ++u) {
        const int f = t + 256 * u;
        if (LAYOUT == KRow) {
            const int k = f / (R / 4);
            const int r = 4 * (f % (R / 4));
            *reinterpret_cast<f32x4*>(s + k * LD + r) = reg[u];
        } else {
            const int r = f / (kBK / 4);
            const int k = 4 * (f % (kBK / 4));
            s[(k + 0) * LD + r] = reg[u].x;
            s[(k + 1) * LD + r] = reg[u].y;
            s[(k + 2) * LD + r] = reg[u].z;
            s[(k + 3) * LD + r] = reg[u].w;
        }
    }
}

template <int WM, int WN>
struct Block {
    static constexpr int BM = 64 * WM;
    static constexpr int BN = 64 * WN;
    static constexpr int LDS_A = kBK * OperandTile<BM>::LD;   // floats per buffer
    static constexpr int LDS_B = kBK * OperandTile<BN>::LD;
    static constexpr int LDS_FLOATS = 2 * (LDS_A + LDS_B);
    static_assert(WM * WN == 4, "four waves per block");
};

// acc[mi][ni] holds the 32 x 32 tile (wave row 32*mi, wave col 32*ni).
struct Acc {
    f32x16 c[2][2];
};

__device__ __forceinline__ void acc_zero(Acc& a)
{
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) a.c[i][j][r] = 0.f;
}

// C_block += A[m-rows, k0:k1] * B[k0:k1, n-cols] for this workgroup.
// A rows beyond `alim` and B columns beyond `blim` read as zero.
// k0, k1 are multiples of kBK.  `lds` must hold Block<WM,WN>::LDS_FLOATS.
template <int WM, int WN, int ALAY, int BLAY>
__device__ __forceinline__ void block_gemm(const float* __restrict__ A, int64_t lda, int alim,
                                           const float* __restrict__ B, int64_t ldb, int blim,
                                           int k0, int k1, float* lds, Acc& acc)
{
    typedef Block<WM, WN> Bk;
    constexpr int BM = Bk::BM, BN = Bk::BN;
    constexpr int LDA = OperandTile<BM>::LD, LDB = OperandTile<BN>::LD;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wy = wave / WN, wx = wave % WN;
    const int kl = lane >> 5, ml = lane & 31;

    f32x4 ra[OperandTile<BM>::PER_THREAD];
    f32x4 rb[OperandTile<BN>::PER_THREAD];
    const int nchunk = (k1 - k0) / kBK;
    if (nchunk <= 0) return;

    load_chunk<BM, ALAY>(A, lda, alim, k0, ra);
    load_chunk<BN, BLAY>(B, ldb, blim, k0, rb);
    store_chunk<BM, ALAY>(lds, ra);
    store_chunk<BN, BLAY>(lds + 2 * Bk::LDS_A, rb);
    __syncthreads();

    for (int c = 0; c < nchunk; ++c) {
        const int buf = c & 1;
        const bool more = (c + 1) < nchunk;
        if (more) {
            load_chunk<BM, ALAY>(A, lda, alim, k0 + (c + 1) * kBK, ra);
            load_chunk<BN, BLAY>(B, ldb, blim, k0 + (c + 1) * kBK, rb);
        }
        const float* sa = lds + buf * Bk::LDS_A + wy * 64 + ml;
        const float* sb = lds + 2 * Bk::LDS_A + buf * Bk::LDS_B + wx * 64 + ml;
#pragma unroll
        for (int kk = 0; kk < kBK; kk += 2) {
            const float a0 = sa[(kk + kl) * LDA];
            const float a1 = sa[(kk + kl) * LDA + 32];
            const float b0 = sb[(kk + kl) * LDB];
            const float b1 = sb[(kk + kl) * LDB + 32];
            acc.c[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc.c[0][0], 0, 0, 0);
            acc.c[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc.c[0][1], 0, 0, 0);
            acc.c[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc.c[1][0], 0, 0, 0);
            acc.c[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc.c[1][1], 0, 0, 0);
        }
        if (more) {
            store_chunk<BM, ALAY>(lds + (buf ^ 1) * Bk::LDS_A, ra);
            store_chunk<BN, BLAY>(lds + 2 * Bk::LDS_A + (buf ^ 1) * Bk::LDS_B, rb);
        }
        __syncthreads();
    }
}

// Row / column (within the block) of accumulator element r of tile (mi, ni)
// for this lane: the v_mfma_f32_32x32x2f32 output layout.
__device__ __forceinline__ int acc_row(int mi, int r)
{
    const int lane = threadIdx.x & 63;
    return 32 * mi + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int ni)
{
    return 32 * ni + (threadIdx.x & 31);
}

// C[(row) * ldc + col] = alpha * acc + beta * C, for block-relative rows
// < rlim and cols < clim, and only where row - col >= diag (pass
// kNoDiag to store the whole block).  beta == 0 does not read C.
constexpr int kNoDiag = -(1 << 30);

template <int WM, int WN>
__device__ __forceinline__ void block_store(float* __restrict__ C, int64_t ldc, int rlim, int clim,
                                            float alpha, float beta, const Acc& acc, int diag = kNoDiag)
{
    const int wave = threadIdx.x >> 6;
    const int wy = wave / WN, wx = wave % WN;
    // rlim and clim are multiples of 64, so a wave's 64 x 64 sub-block is
    // either inside or outside: one wave-uniform test.
    if (wy * 64 >= rlim || wx * 64 >= clim) return;
    float* base = C + (int64_t)(wy * 64) * ldc + wx * 64;
    // all loads first (one wait), then all stores
    float old[2][2][16];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                old[mi][ni][r] = (beta != 0.f) ? base[(int64_t)acc_row(mi, r) * ldc + acc_col(ni)] : 0.f;
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = acc_row(mi, r), col = acc_col(ni);
                if (wy * 64 + row - (wx * 64 + col) < diag) continue;
                base[(int64_t)row * ldc + col] = alpha * acc.c[mi][ni][r] + beta * old[mi][ni][r];
            }
}

}  // namespace bk
