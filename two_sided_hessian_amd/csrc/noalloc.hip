// noalloc.hip -- bakron_solve_noalloc: bakron_solve for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The solve's scratch lives in one file-scope device array, `scratch`, of
// kNoallocScratchBytes; every GPU the library runs on holds its own copy
// until the process ends.  The kernels are bakron_solve's, run unsplit on the
// caller's stream (no library-owned streams, no events), which gives
// bakron_solve's results bit for bit: the split schedule only changes which
// stream runs a part, not the products it sums or their order.
//
// The device address of `scratch` is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept; host code passes
// only that address to the kernels (the array's name is a host-side stand-in
// in host code, not a device address).
#include <map>
#include <mutex>

#include "../../include/bakron.h"
#include "internal.hpp"

namespace {

constexpr size_t kNoallocScratchBytes = (size_t)BAKRON_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of `scratch` on the current device (looked up on the first
// call on each device), or nullptr on failure.
void* scratch_ptr()
{
    static std::mutex mu;
    static std::map<int, void*> ptrs;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    auto it = ptrs.find(dev);
    if (it != ptrs.end()) return it->second;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
    return p;
}

}  // namespace

extern "C" {

int bakron_solve_noalloc(const float* W, int64_t m, int64_t n, const float* L_A, const float* P_A,
                         const float* L_B, const float* P_B, const float* scale, const float* zero,
                         const int32_t* maxq, float* V, uint8_t* codes, float* err, double* objective,
                         hipStream_t stream)
{
    if (m < 0 || n < 0 || m > BAKRON_MAX_DIM || n > BAKRON_MAX_DIM) return BAKRON_ERR_BAD_SIZE;
    if (m == 0 || n == 0) return BAKRON_SUCCESS;
    if (!W || !P_A || !P_B || !scale || !zero || !maxq || !V || !codes) return BAKRON_ERR_NULL_POINTER;
    if (objective && (!L_A || !L_B)) return BAKRON_ERR_NULL_POINTER;
    if (!bk::aligned16(P_A) || !bk::aligned16(P_B)) return BAKRON_ERR_BAD_ARG;
    if (bk::solve_workspace_bytes(m, n, false) > kNoallocScratchBytes) return BAKRON_ERR_TOO_LARGE;
    void* ws = scratch_ptr();
    if (!ws) return BAKRON_ERR_HIP;
    // Nothing in the scratch needs to start at zero: the solve writes every
    // part of it (working weights, errors, stage-1 products, block lists,
    // objective partials) before reading it, as it does with a caller's
    // workspace.
    return bk::solve_enqueue(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective, ws, stream,
                             nullptr, false)
               ? BAKRON_ERR_HIP
               : BAKRON_SUCCESS;
}

}  // extern "C"
