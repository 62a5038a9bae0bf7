// gemm.hpp -- fp32 MFMA block GEMM core for gfx950 (CDNA4).
//
// One workgroup = 4 waves (256 threads) computes a (64*WM) x (64*WN) output
// block; each wave owns one 64 x 64 sub-block as 2 x 2 tiles of
// v_mfma_f32_32x32x2f32 (32 x 32 output, K = 2 per instruction, 16 fp32
// accumulators per lane).  Operands are staged through LDS in K chunks of
// kBK; the next chunk's global loads are issued before the current chunk's
// MFMAs.  Each operand keeps its global orientation in LDS, so global ->
// LDS copies are float4 moves, and K-contiguous operands feed four MFMAs
// per 16-byte LDS read.
//
// Every row/column extent used by the callers is a multiple of 64, so
// per-float4 bounds checks (rows beyond `rlim` read as zero) are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#ifndef BAKRON_KBK
#define BAKRON_KBK 32
#endif
constexpr int kBK = BAKRON_KBK;   // K chunk staged in LDS
constexpr int kPad = 4;   // LDS row padding in floats (keeps 16-byte alignment)

// How an operand is stored in global memory, for operand element (r, k)
// where r runs over the output rows (operand A) or output columns (operand B):
//   RowK: p[r * ld + k]   (K contiguous)  -> LDS [r][k], pitch kBK + kPad
//   KRow: p[k * ld + r]   (r contiguous)  -> LDS [k][r], pitch R + kPad
// Both copies are straight float4 moves (no transposition).
enum Layout { RowK = 0, KRow = 1 };

template <int R, int LAYOUT, int BK = kBK>
struct Operand {
    static constexpr int PITCH = (LAYOUT == RowK) ? (BK + kPad) : (R + kPad);
    static constexpr int FLOATS = (LAYOUT == RowK) ? R * PITCH : BK * PITCH;
    static constexpr int F4 = R * BK / 4;             // float4s per chunk
    static constexpr int PER_THREAD = F4 / 256;       // float4s per thread
    static_assert(F4 % 256 == 0, "tile too small for 256 threads");

    // Global -> registers for one K chunk [k0, k0 + BK); rows >= rlim read 0.
    static __device__ __forceinline__ void load(const float* __restrict__ p, int64_t ld, int rlim, int k0,
                                                f32x4 (&reg)[PER_THREAD])
    {
        const int t = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const int f = t + 256 * u;
            int r, k;
            if (LAYOUT == KRow) {
                k = f / (R / 4);
                r = 4 * (f % (R / 4));
            } else {
                r = f / (BK / 4);
                k = 4 * (f % (BK / 4));
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

    static __device__ __forceinline__ void store(float* __restrict__ s, const f32x4 (&reg)[PER_THREAD])
    {
        const int t = threadIdx.x;
#pragma unroll
        for (int u = 0; u < PER_THREAD; ++u) {
            const int f = t + 256 * u;
            int r, k;
            if (LAYOUT == KRow) {
                k = f / (R / 4);
                r = 4 * (f % (R / 4));
                *reinterpret_cast<f32x4*>(s + k * PITCH + r) = reg[u];
            } else {
                r = f / (BK / 4);
                k = 4 * (f % (BK / 4));
                *reinterpret_cast<f32x4*>(s + r * PITCH + k) = reg[u];
            }
        }
    }

    // MFMA fragment of row `row` for the 8-wide k group starting at kc:
    // element q is k = kc + 4 * (lane >> 5) + q (the same k assignment for
    // both operands, so each v_mfma_f32_32x32x2f32 q contracts k = kc + q
    // and kc + 4 + q).
    static __device__ __forceinline__ f32x4 frag(const float* __restrict__ s, int row, int kc)
    {
        const int kl = (threadIdx.x & 63) >> 5;
        if (LAYOUT == RowK) {
            return *reinterpret_cast<const f32x4*>(s + row * PITCH + kc + 4 * kl);
        } else {
            const float* c = s + (kc + 4 * kl) * PITCH + row;
            f32x4 v;
            v.x = c[0];
            v.y = c[PITCH];
            v.z = c[2 * PITCH];
            v.w = c[3 * PITCH];
            return v;
        }
    }
};

template <int WM, int WN, int ALAY, int BLAY>
struct Gemm {
    static constexpr int BM = 64 * WM;
    static constexpr int BN = 64 * WN;
    typedef Operand<BM, ALAY> OA;
    typedef Operand<BN, BLAY> OB;
    static constexpr int LDS_FLOATS = OA::FLOATS + OB::FLOATS;
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
// k0, k1 are multiples of kBK.  `lds` must hold Gemm<...>::LDS_FLOATS.
// One LDS buffer; the next chunk is prefetched into registers while the
// current one feeds the MFMAs.
template <int WM, int WN, int ALAY, int BLAY>
__device__ __forceinline__ void block_gemm(const float* __restrict__ A, int64_t lda, int alim,
                                           const float* __restrict__ B, int64_t ldb, int blim,
                                           int k0, int k1, float* lds, Acc& acc)
{
    typedef Gemm<WM, WN, ALAY, BLAY> G;
    typedef typename G::OA OA;
    typedef typename G::OB OB;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wy = wave / WN, wx = wave % WN;
    const int ml = lane & 31;
    float* sa = lds;
    float* sb = lds + OA::FLOATS;

    f32x4 ra[OA::PER_THREAD];
    f32x4 rb[OB::PER_THREAD];
    const int nchunk = (k1 - k0) / kBK;
    if (nchunk <= 0) return;

    OA::load(A, lda, alim, k0, ra);
    OB::load(B, ldb, blim, k0, rb);
    OA::store(sa, ra);
    OB::store(sb, rb);
    __syncthreads();

    for (int c = 0; c < nchunk; ++c) {
        const bool more = (c + 1) < nchunk;
        if (more) {
            OA::load(A, lda, alim, k0 + (c + 1) * kBK, ra);
            OB::load(B, ldb, blim, k0 + (c + 1) * kBK, rb);
        }
#pragma unroll
        for (int kc = 0; kc < kBK; kc += 8) {
            const f32x4 a0 = OA::frag(sa, wy * 64 + ml, kc);
            const f32x4 a1 = OA::frag(sa, wy * 64 + 32 + ml, kc);
            const f32x4 b0 = OB::frag(sb, wx * 64 + ml, kc);
            const f32x4 b1 = OB::frag(sb, wx * 64 + 32 + ml, kc);
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
            OA::store(sa, ra);
            OB::store(sb, rb);
            __syncthreads();
        }
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

// C[r * ldc + c] = alpha * acc + beta * C over the wave's 32 x 32 tile,
// only where r - c >= diag.  beta == 0 does not read C.
__device__ __forceinline__ void wave_store32(float* __restrict__ C, int64_t ldc, float alpha, float beta,
                                             const f32x16& acc, int diag = kNoDiag)
{
    const int lane = threadIdx.x & 63;
    const int col = lane & 31;
    float old[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        old[r] = (beta != 0.f) ? C[(int64_t)row * ldc + col] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row - col < diag) continue;
        C[(int64_t)row * ldc + col] = alpha * acc[r] + beta * old[r];
    }
}

// ---------------------------------------- 64 x 64 block, 32 x 32 per wave
//
// For launches with few output tiles: a workgroup computes one 64 x 64
// tile, wave w the 32 x 32 quadrant at rows 32 (w >> 1), columns 32 (w & 1),
// so a launch keeps four waves busy per output tile.  Operands are staged
// through LDS in coalesced chunks of kBK64 that the four waves share; a
// quadrant does only 4 MFMAs per 8 k, so the chunk is deeper than the block
// core's to spread the two barriers of a chunk over more MFMAs.
#ifndef BAKRON_KBK64
#define BAKRON_KBK64 64
#endif
constexpr int kBK64 = BAKRON_KBK64;
constexpr int kLds64 = Operand<64, RowK, kBK64>::FLOATS > Operand<64, KRow, kBK64>::FLOATS
                           ? 2 * Operand<64, RowK, kBK64>::FLOATS
                           : 2 * Operand<64, KRow, kBK64>::FLOATS;

// k0, k1 are multiples of kBK64.
template <int ALAY, int BLAY>
__device__ __forceinline__ void block_gemm64(const float* __restrict__ A, int64_t lda,
                                             const float* __restrict__ B, int64_t ldb, int k0, int k1,
                                             float* lds, f32x16& acc)
{
    typedef Operand<64, ALAY, kBK64> OA;
    typedef Operand<64, BLAY, kBK64> OB;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ml = lane & 31;
    const int ra = 32 * (wave >> 1) + ml, rb = 32 * (wave & 1) + ml;
    float* sa = lds;
    float* sb = lds + OA::FLOATS;
    f32x4 pa[OA::PER_THREAD];
    f32x4 pb[OB::PER_THREAD];
    const int nchunk = (k1 - k0) / kBK64;
    if (nchunk <= 0) return;
    OA::load(A, lda, 64, k0, pa);
    OB::load(B, ldb, 64, k0, pb);
    OA::store(sa, pa);
    OB::store(sb, pb);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
        const bool more = (c + 1) < nchunk;
        if (more) {
            OA::load(A, lda, 64, k0 + (c + 1) * kBK64, pa);
            OB::load(B, ldb, 64, k0 + (c + 1) * kBK64, pb);
        }
#pragma unroll
        for (int kc = 0; kc < kBK64; kc += 8) {
            const f32x4 a = OA::frag(sa, ra, kc);
            const f32x4 b = OB::frag(sb, rb, kc);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
        }
        if (more) {
            __syncthreads();
            OA::store(sa, pa);
            OB::store(sb, pb);
            __syncthreads();
        }
    }
}

}  // namespace bk
