// internal.hpp -- shared host-side declarations of libbakron (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <functional>
#include <vector>

#include "../../include/bakron.h"

namespace bk {

// ------------------------------------------------------------ launches
//
// Every kernel is launched through launch().  With a Prof attached (the
// *_profiled entry points) each launch carries HIP start/stop events
// (hipExtLaunchKernelGGL records them around the kernel itself) and the
// launch's algorithmic flops and bytes; the totals per kernel are read back
// after the stream drains.

// One kind per __global__ function (template instances counted apart), so
// the per-kind statistics line up with a profiler's per-kernel summary.
enum KernelKind {
    KK_COPY_PAD, KK_LEAF, KK_PROP_ROWS, KK_PROP_ROWS_T, KK_PROP_COLS, KK_PROP_COLS_T, KK_OBJ_REDUCE, KK_SCHED,
    KK_F_CLEAR, KK_F_MEAN, KK_F_LOAD, KK_F_DIAG, KK_F_PANEL, KK_F_PANEL_T, KK_F_SYRK_T, KK_F_RIGHT, KK_F_RIGHT_T,
    KK_F_LEFT, KK_F_LEFT_T, KK_F_FINISH, KK_G_LOAD, KK_G_SWEEP, KK_G_UPDATE, KK_G_UPDATE_T, KK_G_OBJ,
    KK_K_SQNORM, KK_K_MOMENT, KK_K_MOMENT_W, KK_PROP_ROWS_FAR, KK_PROP_ROWS_T_FAR, KK_PROP_COLS_FAR,
    KK_PROP_COLS_T_FAR, KK_AD_PREP, KK_AD_QUANT, KK_AD_UPDATE, KK_F_UPDATE, KK_F_U_T, KK_COUNT
};
static_assert(KK_COUNT <= BAKRON_MAX_KERNEL_KINDS, "kernel kinds exceed the ABI's statistics capacity");

const char* kernel_name(int kind);

struct LaunchRec {
    int kind;
    hipEvent_t start, stop;
    double flops, bytes;
};

struct Prof {
    std::vector<LaunchRec> recs;
    bool failed = false;
};

template <typename... KArgs, typename... Args>
inline void launch(Prof* p, int kind, double flops, double bytes, void (*kernel)(KArgs...), dim3 g, dim3 b,
                   hipStream_t s, Args... args)
{
    if (!p) {
        hipLaunchKernelGGL(kernel, g, b, 0, s, static_cast<KArgs>(args)...);
        return;
    }
    LaunchRec r{kind, nullptr, nullptr, flops, bytes};
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
        p->failed = true;
        hipLaunchKernelGGL(kernel, g, b, 0, s, static_cast<KArgs>(args)...);
        return;
    }
    hipExtLaunchKernelGGL(kernel, g, b, 0, s, r.start, r.stop, 0u, static_cast<KArgs>(args)...);
    p->recs.push_back(r);
}

// The same with `shmem` bytes of dynamic LDS reserved for the launch.
template <typename... KArgs, typename... Args>
inline void launch_shm(Prof* p, int kind, double flops, double bytes, void (*kernel)(KArgs...), dim3 g, dim3 b,
                       size_t shmem, hipStream_t s, Args... args)
{
    if (!p) {
        hipLaunchKernelGGL(kernel, g, b, shmem, s, static_cast<KArgs>(args)...);
        return;
    }
    LaunchRec r{kind, nullptr, nullptr, flops, bytes};
    if (hipEventCreate(&r.start) != hipSuccess || hipEventCreate(&r.stop) != hipSuccess) {
        p->failed = true;
        hipLaunchKernelGGL(kernel, g, b, shmem, s, static_cast<KArgs>(args)...);
        return;
    }
    hipExtLaunchKernelGGL(kernel, g, b, shmem, s, r.start, r.stop, 0u, static_cast<KArgs>(args)...);
    p->recs.push_back(r);
}

// A library-owned stream (default priority, non-blocking) for work that a
// call forks off the caller's stream and joins back with events.  A fixed
// pool of kSideSlots streams per device, created on first use and kept for
// the life of the process (so the number of streams never grows with the
// caller's streams).  Calls from different caller streams share the pool:
// their side work is then served in the order it was enqueued, and since
// every wait is on an event recorded before it, no call can wait on another
// call's later work.  nullptr when the stream cannot be created or slot is
// out of range.
constexpr int kSideSlots = 4;
hipStream_t side_stream(int slot);

// Drain the stream, sum the per-launch event times per kernel kind into
// stats (at most max_stats entries, in KernelKind order), release events.
int prof_collect(Prof& p, hipStream_t s, bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats);

constexpr int kTile = 64;            // tile edge of the solve and of the factor's base blocks
constexpr int kMaxDim = BAKRON_MAX_DIM;
constexpr size_t kAlign = 256;       // workspace sub-buffer alignment
constexpr size_t kLeafLdsBytes = 72800;   // LDS of one solve leaf workgroup (k_leaf)

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Factor (factor.hip)
size_t factor_workspace_bytes(int64_t n);
// Leading blocks: when n is a multiple of 64 above 128, the factorisation
// finishes the blocks [0, size)^2 of L and P one after the other, for the
// sizes that factor_leads(n, sizes) lists (smallest first; none otherwise).
// With `leads`, event ev[k] is recorded on `stream` once block size[k] is
// final (events the caller created; sizes not listed are not recorded).
constexpr int kMaxLeads = 16;
struct FactorLeads {
    int count;
    int64_t size[kMaxLeads];
    hipEvent_t ev[kMaxLeads];
};
int factor_leads(int64_t n, int64_t* sizes);
// With `defer`, factor_enqueue appends its stream operations (launches and
// event records, in stream order) to the list instead of issuing them: the
// fused call issues two factors' lists interleaved, so that both chains of
// latency-bound launches start at once.  Each call returns 0 or -1.
using FactorCalls = std::vector<std::function<int()>>;
// `side`: a stream for work of the upper levels that can run beside the
// factor's chain of small launches (see factor_rec); null runs that work in
// order on `stream`, with the same arithmetic.
int factor_enqueue(const float* A, int64_t n, float damp_frac, float* L, float* P, int32_t* info,
                   void* ws, hipStream_t stream, Prof* prof, const FactorLeads* leads = nullptr,
                   FactorCalls* defer = nullptr, hipStream_t side = nullptr);
// Issues two lists one call of each at a time; -1 on the first failure.
int run_interleaved(FactorCalls& a, FactorCalls& b);

// Solve (solve.hip).  With `split`, the far parts of the upper nodes run on
// library-owned streams, ordered against `stream` by events.
size_t solve_workspace_bytes(int64_t m, int64_t n, bool split = true);
// A solve enqueued while its factors are still being computed: for factor
// f (0: A, whose rows and columns are W's columns; 1: B, W's rows), the
// leading block [0, lead[f].size[k])^2 of L and P is final once
// lead[f].ev[k] completes, and everything once full[f] completes.  The solve
// waits for each event just before its first work that needs that block.
struct SolveWait {
    FactorLeads lead[2];
    hipEvent_t full[2];
};
// group_size 0: one grid per row (scale, zero, maxq of length m); otherwise
// a multiple of 64: one grid per (row, group of group_size columns), m x
// ceil(n / group_size) row-major.
int solve_enqueue(const float* W, int64_t m, int64_t n, const float* LA, const float* PA,
                  const float* LB, const float* PB, const float* scale, const float* zero,
                  const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                  void* ws, hipStream_t stream, Prof* prof, bool split = true, const SolveWait* wait = nullptr,
                  int64_t group_size = 0);

// BaKron-antidiagonal: one entry anti-diagonal per step (antidiag.hip)
size_t antidiag_workspace_bytes(int64_t m, int64_t n);
int antidiag_enqueue(const float* W, int64_t m, int64_t n, const float* LA, const float* PA, const float* LB,
                     const float* PB, const float* scale, const float* zero, const int32_t* maxq, float* V,
                     uint8_t* codes, float* err, double* objective, void* ws, hipStream_t stream, Prof* prof);

// One-sided case B = I (gptq.hip)
size_t gptq_workspace_bytes(int64_t m, int64_t n);
int gptq_enqueue(const float* W, int64_t m, int64_t n, const float* LA, const float* PA, const float* scale,
                 const float* zero, const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                 void* ws, hipStream_t stream, Prof* prof, int64_t group_size = 0);

// Kronecker factors from per-sample inputs (kfac.hip)
int sqnorms_enqueue(const float* X, int64_t N, int64_t n, float* out, hipStream_t s, Prof* prof);
int moment_enqueue(const float* X, int64_t N, int64_t n, const float* w, float scale, float* M, hipStream_t s,
                   Prof* prof);

}  // namespace bk
