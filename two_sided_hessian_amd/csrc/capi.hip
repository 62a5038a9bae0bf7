// capi.hip -- extern "C" entry points of libbakron.so (declared in
// include/bakron.h).  Host-side argument checks only; the work is enqueued
// by factor.hip and solve.hip.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/bakron.h"
#include "internal.hpp"

extern "C" {

int bakron_version(void) { return 100; }   // 0.1.0

const char* bakron_strerror(int code)
{
    switch (code) {
    case BAKRON_SUCCESS: return "success";
    case BAKRON_ERR_NULL_POINTER: return "a required pointer is NULL";
    case BAKRON_ERR_BAD_SIZE: return "matrix dimension negative or above BAKRON_MAX_DIM";
    case BAKRON_ERR_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case BAKRON_ERR_BAD_ARG: return "scalar argument out of range";
    case BAKRON_ERR_HIP: return "HIP kernel launch failed";
    case BAKRON_ERR_TOO_LARGE: return "problem needs more scratch than bakron_solve_noalloc's fixed maximum";
    default: return "unknown bakron error code";
    }
}

size_t bakron_factor_workspace_bytes(int64_t n)
{
    if (n <= 0 || n > BAKRON_MAX_DIM) return 0;
    return bk::factor_workspace_bytes(n);
}

size_t bakron_solve_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return 0;
    return bk::solve_workspace_bytes(m, n);
}

static int check_ws(const void* ws, size_t have, size_t need)
{
    if (need == 0) return BAKRON_SUCCESS;
    if (!ws || have < need || (reinterpret_cast<uintptr_t>(ws) % bk::kAlign) != 0) return BAKRON_ERR_WORKSPACE;
    return BAKRON_SUCCESS;
}

// The library stream for a standalone factorisation's right-looking side
// work: slots 2 and 3 in turn, so that two factorisations issued one after
// the other (A and B) use two streams.
static hipStream_t factor_side_stream()
{
    static std::atomic<unsigned> next{0};
    return bk::side_stream(2 + (int)(next.fetch_add(1u, std::memory_order_relaxed) & 1u));
}

int bakron_factor(const float* A, int64_t n, float damp_frac, float* L, float* P, int32_t* info,
                  void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (n < 0 || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (!(damp_frac >= 0.f) || !isfinite(damp_frac)) return BAKRON_ERR_BAD_ARG;
    if (n == 0) return BAKRON_SUCCESS;
    if (!A || !L || !P || !info) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(L) || !bk::aligned16(P)) return BAKRON_ERR_BAD_ARG;
    const int w = check_ws(workspace, workspace_bytes, bk::factor_workspace_bytes(n));
    if (w) return w;
    return bk::factor_enqueue(A, n, damp_frac, L, P, info, workspace, stream, nullptr, nullptr, nullptr,
                              factor_side_stream())
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

int bakron_factor_profiled(const float* A, int64_t n, float damp_frac, float* L, float* P, int32_t* info,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats)
{
    if (!n_stats || (max_stats > 0 && !stats)) return BAKRON_ERR_NULL_POINTER;
    *n_stats = 0;
    if (n < 0 || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (!(damp_frac >= 0.f) || !isfinite(damp_frac)) return BAKRON_ERR_BAD_ARG;
    if (n == 0) return BAKRON_SUCCESS;
    if (!A || !L || !P || !info) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(L) || !bk::aligned16(P)) return BAKRON_ERR_BAD_ARG;
    const int w = check_ws(workspace, workspace_bytes, bk::factor_workspace_bytes(n));
    if (w) return w;
    bk::Prof prof;
    const int rc = bk::factor_enqueue(A, n, damp_frac, L, P, info, workspace, stream, &prof, nullptr, nullptr,
                                      factor_side_stream());
    const int rp = bk::prof_collect(prof, stream, stats, max_stats, n_stats);
    return (rc || rp) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

int bakron_solve(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                 const float* L_B, const float* P_B, const float* scale, const float* zero,
                 const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                 void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(P_A) || !bk::aligned16(P_B)) return BAKRON_ERR_BAD_ARG;
    const int w = check_ws(workspace, workspace_bytes, bk::solve_workspace_bytes(m, n));
    if (w) return w;
    return bk::solve_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective,
                             workspace, stream, nullptr)
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

int bakron_solve_profiled(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                          const float* L_B, const float* P_B, const float* scale, const float* zero,
                          const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                          void* workspace, size_t workspace_bytes, hipStream_t stream,
                          bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats)
{
    if (!n_stats || (max_stats > 0 && !stats)) return BAKRON_ERR_NULL_POINTER;
    *n_stats = 0;
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(P_A) || !bk::aligned16(P_B)) return BAKRON_ERR_BAD_ARG;
    const int w = check_ws(workspace, workspace_bytes, bk::solve_workspace_bytes(m, n));
    if (w) return w;
    bk::Prof prof;
    const int rc = bk::solve_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective,
                                     workspace, stream, &prof);
    const int rp = bk::prof_collect(prof, stream, stats, max_stats, n_stats);
    return (rc || rp) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

int bakron_solve_grouped(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                         const float* L_B, const float* P_B, const float* scale, const float* zero,
                         const int32_t* maxq, int64_t group_size, float* V, uint8_t* codes, float* err,
                         double* objective, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (group_size <= 0 || group_size % bk::kTile != 0) return BAKRON_ERR_BAD_ARG;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(P_A) || !bk::aligned16(P_B)) return BAKRON_ERR_BAD_ARG;
    const int w = check_ws(workspace, workspace_bytes, bk::solve_workspace_bytes(m, n));
    if (w) return w;
    return bk::solve_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective,
                             workspace, stream, nullptr, true, nullptr, group_size)
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

size_t bakron_solve_antidiagonal_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return 0;
    return bk::antidiag_workspace_bytes(m, n);
}

int bakron_solve_antidiagonal(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                              const float* L_B, const float* P_B, const float* scale, const float* zero,
                              const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                              void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    const int w = check_ws(workspace, workspace_bytes, bk::antidiag_workspace_bytes(m, n));
    if (w) return w;
    return bk::antidiag_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective, workspace,
                                stream, nullptr)
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

int bakron_solve_antidiagonal_profiled(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                                       const float* L_B, const float* P_B, const float* scale, const float* zero,
                                       const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream,
                                       bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats)
{
    if (!n_stats || (max_stats > 0 && !stats)) return BAKRON_ERR_NULL_POINTER;
    *n_stats = 0;
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    const int w = check_ws(workspace, workspace_bytes, bk::antidiag_workspace_bytes(m, n));
    if (w) return w;
    bk::Prof prof;
    const int rc = bk::antidiag_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective,
                                        workspace, stream, &prof);
    const int rp = bk::prof_collect(prof, stream, stats, max_stats, n_stats);
    return (rc || rp) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

size_t bakron_quantize_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return 0;
    return bk::align_up(bk::factor_workspace_bytes(n)) + bk::align_up(bk::factor_workspace_bytes(m)) +
           bk::solve_workspace_bytes(m, n);
}

int bakron_quantize(const float* W, int64_t m, int64_t n, const float* A, const float* B, float damp_frac,
                    const float* scale, const float* zero, const int32_t* maxq, float* L_A, float* P_A,
                    int32_t* info_A, float* L_B, float* P_B, int32_t* info_B, float* V, uint8_t* codes,
                    float* err, double* objective, void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (!(damp_frac >= 0.f) || !isfinite(damp_frac)) return BAKRON_ERR_BAD_ARG;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !A || !B || !scale || !zero || !maxq || !L_A || !P_A || !info_A || !L_B || !P_B || !info_B || !V ||
        !codes)
        return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(L_A) || !bk::aligned16(P_A) || !bk::aligned16(L_B) || !bk::aligned16(P_B))
        return BAKRON_ERR_BAD_ARG;
    const int w = check_ws(workspace, workspace_bytes, bakron_quantize_workspace_bytes(m, n));
    if (w) return w;
    char* ws = static_cast<char*>(workspace);
    void* ws_a = ws;
    void* ws_b = ws + bk::align_up(bk::factor_workspace_bytes(n));
    void* ws_s = ws + bk::align_up(bk::factor_workspace_bytes(n)) + bk::align_up(bk::factor_workspace_bytes(m));
    // The factors run on two library-owned streams forked from `stream` (the
    // streams of the solve's depth-0 and depth-1 far parts, which only start
    // once both factors are complete).  Each records an event as each of its
    // leading blocks becomes final; the solve's first work (copies, block
    // lists) starts at once, and each later kernel of it waits for the
    // smallest leading blocks that hold its tiles.
    hipStream_t sa = bk::side_stream(0), sb = bk::side_stream(1);
    bk::SolveWait wait;
    wait.lead[0].count = bk::factor_leads(n, wait.lead[0].size);
    wait.lead[1].count = bk::factor_leads(m, wait.lead[1].size);
    std::vector<hipEvent_t> ev;   // fork, full A, full B, then the lead events
    int rc = (sa && sb) ? BAKRON_SUCCESS : BAKRON_ERR_HIP;
    const int nev = 3 + wait.lead[0].count + wait.lead[1].count;
    for (int k = 0; k < nev && rc == BAKRON_SUCCESS; ++k) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) rc = BAKRON_ERR_HIP;
        else ev.push_back(e);
    }
    if (rc == BAKRON_SUCCESS) {
        wait.full[0] = ev[1];
        wait.full[1] = ev[2];
        int next = 3;
        for (int f = 0; f < 2; ++f)
            for (int k = 0; k < wait.lead[f].count; ++k) wait.lead[f].ev[k] = ev[next++];
        // The two factors' launches are issued interleaved (each is a chain of
        // latency-bound launches; issued one factor after the other, the
        // second chain would start only after the host had issued the first).
        // Their right-looking side work runs on library slots 2 and 3.
        bk::FactorCalls qa, qb;
        if (hipEventRecord(ev[0], stream) != hipSuccess || hipStreamWaitEvent(sa, ev[0], 0) != hipSuccess ||
            hipStreamWaitEvent(sb, ev[0], 0) != hipSuccess ||
            bk::factor_enqueue(A, n, damp_frac, L_A, P_A, info_A, ws_a, sa, nullptr, &wait.lead[0], &qa,
                               bk::side_stream(2)) ||
            bk::factor_enqueue(B, m, damp_frac, L_B, P_B, info_B, ws_b, sb, nullptr, &wait.lead[1], &qb,
                               bk::side_stream(3)) ||
            bk::run_interleaved(qa, qb) || hipEventRecord(ev[1], sa) != hipSuccess ||
            hipEventRecord(ev[2], sb) != hipSuccess ||
            bk::solve_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective, ws_s,
                              stream, nullptr, true, &wait))
            rc = BAKRON_ERR_HIP;
    }
    for (hipEvent_t e : ev)
        if (e) (void)hipEventDestroy(e);
    return rc;
}

static int check_solve_args(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                            const float* L_B, const float* P_B, const float* scale, const float* zero,
                            const int32_t* maxq, float* V, uint8_t* codes, double* objective)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(P_A) || !bk::aligned16(P_B)) return BAKRON_ERR_BAD_ARG;
    return BAKRON_SUCCESS;
}

constexpr int32_t kMaxBatchStreams = 64;

size_t bakron_solve_batch_workspace_bytes(const bakron_layer* layers, int32_t count, int32_t n_streams)
{
    if (!layers || count <= 0 || n_streams <= 0 || n_streams > kMaxBatchStreams) return 0;
    size_t total = 0;
    for (int32_t s = 0; s < n_streams; ++s) {
        size_t need = 0;
        for (int32_t k = s; k < count; k += n_streams) {
            const bakron_layer& L = layers[k];
            if (L.m > 0 && L.n > 0 && L.m <= BAKRON_MAX_DIM && L.n <= BAKRON_MAX_DIM)
                need = std::max(need, bk::solve_workspace_bytes(L.m, L.n, false));
        }
        total += bk::align_up(need);
    }
    return total;
}

int bakron_solve_batch(const bakron_layer* layers, int32_t count, void* workspace, size_t workspace_bytes,
                       const hipStream_t* streams, int32_t n_streams)
{
    if (count < 0) return BAKRON_ERR_BAD_SIZE;
    if (count == 0) return BAKRON_SUCCESS;
    if (!layers || !streams) return BAKRON_ERR_NULL_POINTER;
    if (n_streams <= 0 || n_streams > kMaxBatchStreams) return BAKRON_ERR_BAD_ARG;
    for (int32_t k = 0; k < count; ++k) {
        const bakron_layer& L = layers[k];
        const int c = check_solve_args(L.W, L.m, L.n, L.L_A, L.P_A, L.L_B, L.P_B, L.scale, L.zero, L.maxq, L.V,
                                       L.codes, L.objective);
        if (c) return c;
    }
    const size_t need = bakron_solve_batch_workspace_bytes(layers, count, n_streams);
    const int w = check_ws(workspace, workspace_bytes, need);
    if (w) return w;
    // slice s starts after the slices of streams 0 .. s-1
    char* base = static_cast<char*>(workspace);
    for (int32_t s = 0; s < n_streams && s < count; ++s) {
        size_t slice = 0;
        for (int32_t k = s; k < count; k += n_streams) {
            const bakron_layer& L = layers[k];
            if (L.m > 0 && L.n > 0) slice = std::max(slice, bk::solve_workspace_bytes(L.m, L.n, false));
        }
        for (int32_t k = s; k < count; k += n_streams) {
            const bakron_layer& L = layers[k];
            if (L.m == 0 || L.n == 0) continue;
            if (bk::solve_enqueue(L.W, L.m, L.n, L.L_A, L.P_A, L.L_B, L.P_B, L.scale, L.zero, L.maxq, L.V, L.codes,
                                  L.err, L.objective, base, streams[s], nullptr, false))
                return BAKRON_ERR_HIP;
        }
        base += bk::align_up(slice);
    }
    return BAKRON_SUCCESS;
}

size_t bakron_gptq_workspace_bytes(int64_t m, int64_t n)
{
    if (m <= 0 || n <= 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return 0;
    return bk::gptq_workspace_bytes(m, n);
}

static int check_gptq(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A, const float* scale,
                      const float* zero, const int32_t* maxq, float* V, uint8_t* codes, double* objective,
                      void* workspace, size_t workspace_bytes)
{
    if (!W || !P_A || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && !L_A) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(P_A)) return BAKRON_ERR_BAD_ARG;
    return check_ws(workspace, workspace_bytes, bk::gptq_workspace_bytes(m, n));
}

int bakron_gptq(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A, const float* scale,
                const float* zero, const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                void* workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    const int c = check_gptq(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, objective, workspace, workspace_bytes);
    if (c) return c;
    return bk::gptq_enqueue(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, err, objective, workspace, stream,
                            nullptr)
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

int bakron_gptq_grouped(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                        const float* scale, const float* zero, const int32_t* maxq, int64_t group_size, float* V,
                        uint8_t* codes, float* err, double* objective, void* workspace, size_t workspace_bytes,
                        hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (group_size <= 0 || group_size % bk::kTile != 0) return BAKRON_ERR_BAD_ARG;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    const int c = check_gptq(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, objective, workspace, workspace_bytes);
    if (c) return c;
    return bk::gptq_enqueue(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, err, objective, workspace, stream,
                            nullptr, group_size)
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

int bakron_gptq_profiled(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                         const float* scale, const float* zero, const int32_t* maxq, float* V, uint8_t* codes,
                         float* err, double* objective, void* workspace, size_t workspace_bytes, hipStream_t stream,
                         bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats)
{
    if (!n_stats || (max_stats > 0 && !stats)) return BAKRON_ERR_NULL_POINTER;
    *n_stats = 0;
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    const int c = check_gptq(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, objective, workspace, workspace_bytes);
    if (c) return c;
    bk::Prof prof;
    const int rc = bk::gptq_enqueue(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, err, objective, workspace,
                                    stream, &prof);
    const int rp = bk::prof_collect(prof, stream, stats, max_stats, n_stats);
    return (rc || rp) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

static int check_samples(const float* X, int64_t N, int64_t n)
{
    if (N < 0 || n < 0 || n > BAKRON_MAX_DIM || N > ((int64_t)1 << 40)) return BAKRON_ERR_BAD_SIZE;
    if (n == 0) return BAKRON_SUCCESS;
    if (!X) return BAKRON_ERR_NULL_POINTER;
    if (n % 4 != 0 || !bk::aligned16(X)) return BAKRON_ERR_BAD_ARG;
    return BAKRON_SUCCESS;
}

int bakron_row_sqnorms(const float* X, int64_t N, int64_t n, float* out, hipStream_t stream)
{
    const int c = check_samples(X, N, n);
    if (c || n == 0 || N == 0) return c;
    if (!out) return BAKRON_ERR_NULL_POINTER;
    return bk::sqnorms_enqueue(X, N, n, out, stream, nullptr) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

int bakron_moment(const float* X, int64_t N, int64_t n, const float* w, float scale, float* M, hipStream_t stream)
{
    const int c = check_samples(X, N, n);
    if (c || n == 0) return c;
    if (!M) return BAKRON_ERR_NULL_POINTER;
    if (!isfinite(scale)) return BAKRON_ERR_BAD_ARG;
    return bk::moment_enqueue(X, N, n, w, scale, M, stream, nullptr) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

int bakron_moment_profiled(const float* X, int64_t N, int64_t n, const float* w, float scale, float* M,
                           hipStream_t stream, bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats)
{
    if (!n_stats || (max_stats > 0 && !stats)) return BAKRON_ERR_NULL_POINTER;
    *n_stats = 0;
    const int c = check_samples(X, N, n);
    if (c || n == 0) return c;
    if (!M) return BAKRON_ERR_NULL_POINTER;
    if (!isfinite(scale)) return BAKRON_ERR_BAD_ARG;
    bk::Prof prof;
    const int rc = bk::moment_enqueue(X, N, n, w, scale, M, stream, &prof);
    const int rp = bk::prof_collect(prof, stream, stats, max_stats, n_stats);
    return (rc || rp) ? BAKRON_ERR_HIP : BAKRON_SUCCESS;
}

}  // extern "C"

namespace bk {

const char* kernel_name(int kind)
{
    static const char* const names[KK_COUNT] = {
        "k_copy_pad", "k_leaf", "k_prop_rows", "k_prop_rows_t", "k_prop_cols", "k_prop_cols_t", "k_obj_reduce",
        "k_sched", "k_clear_info", "k_diag_mean", "k_load_damped", "k_f_diag", "k_f_panel", "k_f_tile<0>",
        "k_f_tile<1>", "k_f_right", "k_f_tile<2>", "k_f_left", "k_f_tile<3>", "k_f_finish", "k_gptq_load",
        "k_gptq_sweep", "k_gptq_update", "k_gptq_update_t", "k_gptq_obj", "k_row_sqnorms", "k_moment<false>",
        "k_moment<true>", "k_prop_rows_far", "k_prop_rows_t_far", "k_prop_cols_far", "k_prop_cols_t_far",
        "k_ad_prep", "k_ad_quant", "k_ad_update", "k_f_update", "k_f_tile<4>"};
    return (kind >= 0 && kind < KK_COUNT) ? names[kind] : "?";
}

hipStream_t side_stream(int slot)
{
    // kSideSlots streams per device, created on first use: the pool does not
    // grow with the number of caller streams.
    static std::mutex mu;
    static std::map<std::pair<int, int>, hipStream_t> table;
    if (slot < 0 || slot >= kSideSlots) return nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    hipStream_t& st = table[std::make_pair(dev, slot)];
    if (!st && hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) st = nullptr;
    return st;
}

int prof_collect(Prof& p, hipStream_t s, bakron_kernel_stat* stats, int32_t max_stats, int32_t* n_stats)
{
    int rc = (hipStreamSynchronize(s) == hipSuccess && !p.failed) ? 0 : -1;
    bakron_kernel_stat acc[KK_COUNT];
    for (int k = 0; k < KK_COUNT; ++k) acc[k] = bakron_kernel_stat{kernel_name(k), 0, 0.0, 0.0, 0.0};
    for (const LaunchRec& r : p.recs) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) rc = -1;
        acc[r.kind].launches += 1;
        acc[r.kind].total_ms += ms;
        acc[r.kind].alg_flops += r.flops;
        acc[r.kind].alg_bytes += r.bytes;
        (void)hipEventDestroy(r.start);
        (void)hipEventDestroy(r.stop);
    }
    p.recs.clear();
    int w = 0;
    for (int k = 0; k < KK_COUNT && w < max_stats; ++k)
        if (acc[k].launches > 0) stats[w++] = acc[k];
    *n_stats = w;
    return rc;
}

}  // namespace bk
