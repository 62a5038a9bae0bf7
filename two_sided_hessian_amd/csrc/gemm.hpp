// gemm.hpp -- fp32 MFMA block GEMM core for gfx950 (CDNA4).
//
// One workgroup = 4 waves (256 threads) computes a (64*WM) x (64*WN) output
// block; each wave owns one 64 x 64 sub-block as 2 x 2 tiles of
// v_mfma_f32_32x32x2f32 (32 x 32 output, K = 2 per instruction, 16 fp32
// accumulators per lane).  Operands are staged through LDS in K chunks of
// kBK with gfx950's direct global -> LDS loads (global_load_lds_dwordx4:
// each lane's 16 bytes go straight to LDS, no register round trip) into two
// LDS buffers, so the next chunk streams in while the current one feeds the
// MFMAs and a chunk costs one barrier.  Each operand keeps its global
// orientation in LDS; K-contiguous operands feed four MFMAs per 16-byte LDS
// read.
//
// Every row/column extent used by the callers is a multiple of 64, so
// limits (rows beyond `rlim` are not needed) are handled per 64 rows.
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

typedef __attribute__((address_space(1))) const void* global_cptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

// Direct staging of one kBK chunk: one wave instruction fills 1 KB of LDS,
// lane L the 16 bytes at 16 L, so the LDS image is fixed by which global
// float4 each lane fetches.
//   RowK: an instruction covers 8 rows x 32 k (rows 128 bytes apart, no
//         padding); row r's k-quad u sits in 16-byte slot u ^ (r & 7), so
//         the eight rows of a fragment read hit eight different slots.
//   KRow: an instruction covers 256 / R k-rows of R floats, pitch R.
// Rows >= rlim are not needed by the caller (they only reach outputs it
// does not store): RowK skips their instructions (rlim is a multiple of 64,
// so the test is wave-uniform); KRow fetches an in-range column in their
// place.  Either way every global address stays inside the operand.
template <int R, int LAYOUT>
struct Direct {
    static constexpr int FLOATS = R * kBK;
    static constexpr int INSTR = FLOATS / 256;     // wave instructions per chunk
    static constexpr int PER_WAVE = INSTR / 4;
    static_assert(kBK == 32 && INSTR % 4 == 0, "direct staging assumes 32-deep chunks, R >= 32");

    static __device__ __forceinline__ void issue(const float* __restrict__ p, int64_t ld, int rlim, int k0, float* s)
    {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3);   // (within a 4-wave group)
#pragma unroll
        for (int i = 0; i < PER_WAVE; ++i) {
            const int q = wave + 4 * i;
            const float* src;
            if (LAYOUT == RowK) {
                if (8 * q >= rlim) continue;
                const int r = 8 * q + (lane >> 3);
                src = p + (int64_t)r * ld + k0 + 4 * ((lane & 7) ^ (r & 7));
            } else {
                const int f = 64 * q + lane;
                int r = 4 * (f % (R / 4));
                if (R > 64) r = min(r, rlim - 4);
                src = p + (int64_t)(k0 + f / (R / 4)) * ld + r;
            }
            __builtin_amdgcn_global_load_lds((global_cptr)src, (lds_ptr)(s + 256 * q), 16, 0, 0);
        }
    }

    // Same fragment as Operand::frag: element q is k = kc + 4 (lane >> 5) + q.
    static __device__ __forceinline__ f32x4 frag(const float* __restrict__ s, int row, int kc)
    {
        const int kl = (threadIdx.x & 63) >> 5;
        if (LAYOUT == RowK) {
            return *reinterpret_cast<const f32x4*>(s + row * kBK + 4 * (((kc >> 2) + kl) ^ (row & 7)));
        } else {
            const float* c = s + (kc + 4 * kl) * R + row;
            f32x4 v;
            v.x = c[0];
            v.y = c[R];
            v.z = c[2 * R];
            v.w = c[3 * R];
            return v;
        }
    }
};

// Direct loads count against vmcnt until their data is in LDS.
__device__ __forceinline__ void wait_direct_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// The same, leaving one 64-row chunk of both operands in flight: each wave
// issues Direct<64, *>::PER_WAVE = 2 loads per operand and chunk, and loads
// complete in order.
#ifndef BAKRON_TILE_PREFETCH2
#define BAKRON_TILE_PREFETCH2 1
#endif
__device__ __forceinline__ void wait_direct_loads_but_one_chunk64()
{
    asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
}

template <int WM, int WN, int ALAY, int BLAY>
struct Gemm {
    static constexpr int BM = 64 * WM;
    static constexpr int BN = 64 * WN;
    typedef Direct<BM, ALAY> OA;
    typedef Direct<BN, BLAY> OB;
    static constexpr int BUF = OA::FLOATS + OB::FLOATS;
    static constexpr int LDS_FLOATS = 2 * BUF;   // two chunk buffers
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
// A rows beyond `alim` and B columns beyond `blim` are not needed (their
// outputs are garbage: store with the same limits).  k0, k1 are multiples
// of kBK.  `lds` must hold Gemm<...>::LDS_FLOATS; it is free again when
// this returns.
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
    const int nchunk = (k1 - k0) / kBK;
    if (nchunk <= 0) return;

    OA::issue(A, lda, alim, k0, lds);
    OB::issue(B, ldb, blim, k0, lds + OA::FLOATS);
    for (int c = 0; c < nchunk; ++c) {
        // chunk c is in LDS for every wave, and every wave is done with
        // chunk c - 1, whose buffer the next issue overwrites
        wait_direct_loads();
        __syncthreads();
        if (c + 1 < nchunk) {
            float* nb = lds + ((c + 1) & 1) * G::BUF;
            OA::issue(A, lda, alim, k0 + (c + 1) * kBK, nb);
            OB::issue(B, ldb, blim, k0 + (c + 1) * kBK, nb + OA::FLOATS);
        }
        const float* sa = lds + (c & 1) * G::BUF;
        const float* sb = sa + OA::FLOATS;
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
    }
    __syncthreads();
}

// block_gemm for one half of a 512-thread workgroup whose two 4-wave halves
// work on two blocks at once (threads 0 - 255 and 256 - 511, each with its
// own `lds`).  Every barrier is shared: both halves run nmax chunk steps,
// nmax the larger of their chunk counts, and a half with fewer chunks waits
// out the rest.  The MFMAs of a block are those of block_gemm, in the same
// order.
template <int WM, int WN, int ALAY, int BLAY>
__device__ __forceinline__ void dual_block_gemm(const float* __restrict__ A, int64_t lda, int alim,
                                                const float* __restrict__ B, int64_t ldb, int blim,
                                                int k0, int k1, int nmax, float* lds, Acc& acc)
{
    typedef Gemm<WM, WN, ALAY, BLAY> G;
    typedef typename G::OA OA;
    typedef typename G::OB OB;
    const int lane = threadIdx.x & 63;
    const int wave = (threadIdx.x >> 6) & 3;
    const int wy = wave / WN, wx = wave % WN;
    const int ml = lane & 31;
    const int nchunk = k1 > k0 ? (k1 - k0) / kBK : 0;
    if (nchunk > 0) {
        OA::issue(A, lda, alim, k0, lds);
        OB::issue(B, ldb, blim, k0, lds + OA::FLOATS);
    }
    for (int c = 0; c < nmax; ++c) {
        wait_direct_loads();
        __syncthreads();
        if (c + 1 < nchunk) {
            float* nb = lds + ((c + 1) & 1) * G::BUF;
            OA::issue(A, lda, alim, k0 + (c + 1) * kBK, nb);
            OB::issue(B, ldb, blim, k0 + (c + 1) * kBK, nb + OA::FLOATS);
        }
        if (c < nchunk) {
            const float* sa = lds + (c & 1) * G::BUF;
            const float* sb = sa + OA::FLOATS;
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
        }
    }
    __syncthreads();
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
    const int wave = __builtin_amdgcn_readfirstlane((threadIdx.x >> 6) & 3);   // (within a 4-wave group)
    const int wy = wave / WN, wx = wave % WN;
    // rlim and clim are multiples of 64, so a wave's 64 x 64 sub-block is
    // either inside or outside: one wave-uniform test.
    if (wy * 64 >= rlim || wx * 64 >= clim) return;
    float* base = C + (int64_t)(wy * 64) * ldc + wx * 64;   // wave-uniform
    const uint32_t ld32 = (uint32_t)ldc;                      // 64 ldc < 2^32
    // one 32 x 32 tile at a time: its 16 loads, one wait, its 16 stores
    // (keeps the epilogue's registers below the main loop's)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
            float old[16];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                old[r] = (beta != 0.f) ? base[(uint32_t)acc_row(mi, r) * ld32 + (uint32_t)acc_col(ni)] : 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = acc_row(mi, r), col = acc_col(ni);
                if (wy * 64 + row - (wx * 64 + col) < diag) continue;
                base[(uint32_t)row * ld32 + (uint32_t)col] = alpha * acc.c[mi][ni][r] + beta * old[r];
            }
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
// so a launch keeps four waves busy per output tile.  A quadrant does only
// 4 MFMAs per 8 k.  With a K-contiguous A operand the chunks are staged by
// direct loads into two buffers (one barrier per kBK chunk); with both
// operands K-major (four scalar LDS reads per fragment on each side) the
// register-staged copy in deeper chunks of kBK64 measured faster.
#ifndef BAKRON_KBK64
#define BAKRON_KBK64 64
#endif
constexpr int kBK64 = BAKRON_KBK64;
constexpr int kLdsStaged64 = Operand<64, RowK, kBK64>::FLOATS > Operand<64, KRow, kBK64>::FLOATS
                                 ? 2 * Operand<64, RowK, kBK64>::FLOATS
                                 : 2 * Operand<64, KRow, kBK64>::FLOATS;
constexpr int kLdsDirect64 = 2 * 2 * Direct<64, RowK>::FLOATS;
constexpr int kLds64 = kLdsStaged64 > kLdsDirect64 ? kLdsStaged64 : kLdsDirect64;

// k0, k1 are multiples of kBK64; `lds` holds kLds64 floats and is free
// again when this returns.
template <int ALAY, int BLAY>
__device__ __forceinline__ void block_gemm64(const float* __restrict__ A, int64_t lda,
                                             const float* __restrict__ B, int64_t ldb, int k0, int k1,
                                             float* lds, f32x16& acc)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ml = lane & 31;
    const int ra = 32 * (wave >> 1) + ml, rb = 32 * (wave & 1) + ml;
    if (ALAY == RowK) {
        typedef Direct<64, ALAY> OA;
        typedef Direct<64, BLAY> OB;
        constexpr int BUF = OA::FLOATS + OB::FLOATS;
        static_assert(OA::PER_WAVE + OB::PER_WAVE == 4, "vmcnt(4) leaves one chunk of both operands in flight");
        const int nchunk = (k1 - k0) / kBK;
        if (nchunk <= 0) return;
        // the first two chunks are issued together (both buffers are free), so
        // a launch with one tile per CU waits for one load latency, not two
        OA::issue(A, lda, 64, k0, lds);
        OB::issue(B, ldb, 64, k0, lds + OA::FLOATS);
        if (BAKRON_TILE_PREFETCH2 && nchunk > 1) {
            OA::issue(A, lda, 64, k0 + kBK, lds + BUF);
            OB::issue(B, ldb, 64, k0 + kBK, lds + BUF + OA::FLOATS);
        }
        for (int c = 0; c < nchunk; ++c) {
            if (BAKRON_TILE_PREFETCH2 && c == 0 && nchunk > 1) {
                // chunk 1 may still be in flight; no LDS access precedes this
                // one in the call, so a bare barrier (no fence, which would
                // wait for every load) is enough to publish chunk 0
                wait_direct_loads_but_one_chunk64();
                __builtin_amdgcn_s_barrier();
            } else {
                wait_direct_loads();
                __syncthreads();
            }
            if (c + 1 < nchunk && !(BAKRON_TILE_PREFETCH2 && c == 0)) {
                float* nb = lds + ((c + 1) & 1) * BUF;
                OA::issue(A, lda, 64, k0 + (c + 1) * kBK, nb);
                OB::issue(B, ldb, 64, k0 + (c + 1) * kBK, nb + OA::FLOATS);
            }
            const float* sa = lds + (c & 1) * BUF;
            const float* sb = sa + OA::FLOATS;
#pragma unroll
            for (int kc = 0; kc < kBK; kc += 8) {
                const f32x4 a = OA::frag(sa, ra, kc);
                const f32x4 b = OB::frag(sb, rb, kc);
#pragma unroll
                for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[q], b[q], acc, 0, 0, 0);
            }
        }
        __syncthreads();
        return;
    }
    typedef Operand<64, ALAY, kBK64> OA;
    typedef Operand<64, BLAY, kBK64> OB;
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
        __syncthreads();
        if (more) {
            OA::store(sa, pa);
            OB::store(sb, pb);
            __syncthreads();
        }
    }
}

}  // namespace bk
