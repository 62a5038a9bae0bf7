// Host-sanitizer driver for the C ABI of libbakron (include/bakron.h), built
// with AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
// by tests/test_sanitizers.py and run on the CPU.  It exercises the paths
// that run before any device call: the workspace sizes over many shapes,
// every host-side argument error, the batch descriptors' checks, the fixed
// scratch limit of the no-allocation call, the error strings.  Pointers are
// fake (never dereferenced: every call returns from its host checks).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/bakron.h"

static int fails = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            printf("FAIL line %d: %s\n", __LINE__, #cond);             \
            ++fails;                                                   \
        }                                                              \
    } while (0)

int main()
{
    void* f = reinterpret_cast<void*>(4096);
    float* ff = static_cast<float*>(f);
    const int32_t* fi = static_cast<const int32_t*>(f);
    uint8_t* fc = static_cast<uint8_t*>(f);
    int32_t* fo = static_cast<int32_t*>(f);
    const size_t big = (size_t)1 << 40;
    // sizes over a sweep of shapes, including the largest dimension
    const int64_t dims[] = {0, 1, 2, 63, 64, 65, 127, 128, 129, 1000, 4096, 14336, 65536, 65537};
    for (int64_t m : dims)
        for (int64_t n : dims) {
            const bool ok = m > 0 && n > 0 && m <= BAKRON_MAX_DIM && n <= BAKRON_MAX_DIM;
            EXPECT((bakron_solve_workspace_bytes(m, n) > 0) == ok);
            EXPECT((bakron_gptq_workspace_bytes(m, n) > 0) == ok);
            EXPECT((bakron_quantize_workspace_bytes(m, n) > 0) == ok);
            EXPECT((bakron_solve_antidiagonal_workspace_bytes(m, n) > 0) == ok);
            EXPECT(bakron_solve_workspace_bytes(m, n) % 256 == 0);
        }
    for (int64_t n : dims) EXPECT((bakron_factor_workspace_bytes(n) > 0) == (n > 0 && n <= BAKRON_MAX_DIM));
    for (int c = -10; c <= 2; ++c) EXPECT(bakron_strerror(c) != nullptr && strlen(bakron_strerror(c)) > 0);
    EXPECT(bakron_version() > 0);
    // factor
    EXPECT(bakron_factor(ff, -1, 0.01f, ff, ff, fo, f, big, nullptr) == BAKRON_ERR_BAD_SIZE);
    EXPECT(bakron_factor(ff, 8, -1.f, ff, ff, fo, f, big, nullptr) == BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_factor(nullptr, 8, 0.01f, ff, ff, fo, f, big, nullptr) == BAKRON_ERR_NULL_POINTER);
    EXPECT(bakron_factor(ff, 8, 0.01f, ff, ff, fo, f, 16, nullptr) == BAKRON_ERR_WORKSPACE);
    EXPECT(bakron_factor(ff, 0, 0.01f, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == BAKRON_SUCCESS);
    // solve, grouped solve, antidiagonal, no-allocation solve
    EXPECT(bakron_solve(ff, 64, 64, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, f, 100, nullptr) ==
           BAKRON_ERR_WORKSPACE);
    EXPECT(bakron_solve(ff, 64, -2, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, f, big, nullptr) ==
           BAKRON_ERR_BAD_SIZE);
    EXPECT(bakron_solve(ff, 64, 64, nullptr, ff, nullptr, ff, ff, ff, fi, ff, fc, nullptr, (double*)f, f, big,
                        nullptr) == BAKRON_ERR_NULL_POINTER);
    EXPECT(bakron_solve_grouped(ff, 64, 200, ff, ff, ff, ff, ff, ff, fi, 96, ff, fc, nullptr, nullptr, f, big,
                                nullptr) == BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_solve_grouped(ff, 64, 200, ff, ff, ff, ff, ff, ff, fi, 0, ff, fc, nullptr, nullptr, f, big,
                                nullptr) == BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_gptq_grouped(ff, 64, 200, ff, ff, ff, ff, fi, 32, ff, fc, nullptr, nullptr, f, big, nullptr) ==
           BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_solve_antidiagonal(ff, 64, 64, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, f, 64,
                                     nullptr) == BAKRON_ERR_WORKSPACE);
    EXPECT(bakron_solve_antidiagonal(nullptr, 64, 64, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, f, big,
                                     nullptr) == BAKRON_ERR_NULL_POINTER);
    EXPECT(bakron_solve_noalloc(ff, 8192, 8192, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, nullptr) ==
           BAKRON_ERR_TOO_LARGE);
    EXPECT(bakron_solve_noalloc(ff, 65536, 65536, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, nullptr) ==
           BAKRON_ERR_TOO_LARGE);
    EXPECT(bakron_solve_noalloc(ff, 65537, 64, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, nullptr) ==
           BAKRON_ERR_BAD_SIZE);
    EXPECT(bakron_solve_noalloc(ff, 64, 64, ff, nullptr, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, nullptr) ==
           BAKRON_ERR_NULL_POINTER);
    // quantize and gptq
    EXPECT(bakron_quantize(ff, 64, 64, ff, ff, -0.5f, ff, ff, fi, ff, ff, fo, ff, ff, fo, ff, fc, nullptr, nullptr,
                           f, big, nullptr) == BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_quantize(ff, 64, 64, ff, ff, 0.01f, ff, ff, fi, ff, ff, fo, ff, ff, fo, ff, fc, nullptr, nullptr,
                           f, 1000, nullptr) == BAKRON_ERR_WORKSPACE);
    EXPECT(bakron_gptq(ff, 64, 64, ff, nullptr, ff, ff, fi, ff, fc, nullptr, nullptr, f, big, nullptr) ==
           BAKRON_ERR_NULL_POINTER);
    // batches: descriptors are all checked before anything runs
    bakron_layer L[3];
    for (bakron_layer& l : L) {
        memset(&l, 0, sizeof(l));
        l.W = l.P_A = l.P_B = l.scale = l.zero = ff;
        l.maxq = fi;
        l.V = ff;
        l.codes = fc;
        l.m = 100;
        l.n = 70;
    }
    L[2].P_A = nullptr;
    hipStream_t st[2] = {nullptr, nullptr};
    EXPECT(bakron_solve_batch(L, 3, f, big, st, 2) == BAKRON_ERR_NULL_POINTER);
    EXPECT(bakron_solve_batch(L, 2, f, 10, st, 2) == BAKRON_ERR_WORKSPACE);
    EXPECT(bakron_solve_batch(L, 2, f, big, st, 65) == BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_solve_batch_workspace_bytes(L, 2, 1) == bakron_solve_batch_workspace_bytes(L, 1, 1));
    EXPECT(bakron_solve_batch_workspace_bytes(nullptr, 2, 1) == 0);
    // sample moments
    EXPECT(bakron_moment(ff, 16, 6, nullptr, 1.f, ff, nullptr) == BAKRON_ERR_BAD_ARG);
    EXPECT(bakron_row_sqnorms(ff, -1, 8, ff, nullptr) == BAKRON_ERR_BAD_SIZE);
    // profiled entry points
    bakron_kernel_stat stats[BAKRON_MAX_KERNEL_KINDS];
    int32_t ns = -1;
    EXPECT(bakron_solve_profiled(nullptr, 64, 64, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, f, big,
                                 nullptr, stats, BAKRON_MAX_KERNEL_KINDS, &ns) == BAKRON_ERR_NULL_POINTER && ns == 0);
    EXPECT(bakron_solve_antidiagonal_profiled(ff, -1, 64, ff, ff, ff, ff, ff, ff, fi, ff, fc, nullptr, nullptr, f,
                                              big, nullptr, stats, BAKRON_MAX_KERNEL_KINDS,
                                              &ns) == BAKRON_ERR_BAD_SIZE);
    printf(fails ? "ABI SANITIZE FAIL (%d)\n" : "ABI SANITIZE OK\n", fails);
    return fails ? 1 : 0;
}
