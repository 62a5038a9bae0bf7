"""The C ABI of libbakron.so, checked on the CPU: the library loads, exports
every function include/bakron.h declares, and rejects bad arguments on the
host (these paths return before any device call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bakron.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bakron_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def B():
    import two_sided_hessian_amd as B
    if not os.path.exists(B.LIB_PATH):
        from two_sided_hessian_amd import build
        build.build()
    return B


def test_header_declares_the_api():
    names = _declared()
    assert names == sorted(["bakron_version", "bakron_strerror", "bakron_factor_workspace_bytes",
                            "bakron_factor", "bakron_solve_workspace_bytes", "bakron_solve",
                            "bakron_factor_profiled", "bakron_solve_profiled",
                            "bakron_gptq_workspace_bytes", "bakron_gptq", "bakron_gptq_profiled",
                            "bakron_row_sqnorms", "bakron_moment", "bakron_moment_profiled",
                            "bakron_solve_batch_workspace_bytes", "bakron_solve_batch",
                            "bakron_quantize_workspace_bytes", "bakron_quantize", "bakron_solve_noalloc",
                            "bakron_solve_grouped", "bakron_gptq_grouped",
                            "bakron_solve_antidiagonal_workspace_bytes", "bakron_solve_antidiagonal",
                            "bakron_solve_antidiagonal_profiled"])


def test_library_exports_every_declared_symbol(B):
    L = B.lib()
    from two_sided_hessian_amd._binding import SIGNATURES
    for name in _declared():
        assert hasattr(L, name), name
        assert name in SIGNATURES, name


def test_header_constants_match_binding(B):
    src = open(HEADER).read()
    from two_sided_hessian_amd import _binding as bb
    for k in ("BAKRON_SUCCESS", "BAKRON_ERR_NULL_POINTER", "BAKRON_ERR_BAD_SIZE", "BAKRON_ERR_WORKSPACE",
              "BAKRON_ERR_BAD_ARG", "BAKRON_ERR_HIP", "BAKRON_ERR_TOO_LARGE", "BAKRON_MAX_DIM",
              "BAKRON_MAX_KERNEL_KINDS"):
        v = re.search(r"#define\s+%s\s+\(?(-?\d+)\)?" % k, src).group(1)
        assert int(v) == getattr(bb, k), k


def test_host_only_calls(B):
    assert B.version() == 100
    assert "workspace" in B.strerror(-3)
    assert "unknown" in B.strerror(12345)
    assert B.factor_workspace_bytes(0) == 0
    # the fused call's workspace holds both factor workspaces and the solve's
    m, n = 256, 320
    assert B.quantize_workspace_bytes(m, n) >= (B.factor_workspace_bytes(n) + B.factor_workspace_bytes(m)
                                                + B.solve_workspace_bytes(m, n))
    assert B.quantize_workspace_bytes(0, n) == 0
    assert B.solve_workspace_bytes(0, 5) == 0
    assert B.solve_workspace_bytes(-1, 5) == 0
    # three m x n float32 matrices at least, plus padded copies when ragged
    assert B.solve_workspace_bytes(128, 128) >= 3 * 128 * 128 * 4
    assert B.solve_workspace_bytes(100, 70) >= 3 * 128 * 128 * 4 + 128 * 128 * 4 + 128 * 128 * 4
    assert B.factor_workspace_bytes(8192) >= 4096 * 4096 * 4
    # one n2 x n1 product buffer per depth of the recursion (8192: 4096^2 + 2048^2 + ... + 128^2 floats)
    assert B.factor_workspace_bytes(8192) >= 4 * sum((4096 >> d) ** 2 for d in range(6))
    assert B.factor_workspace_bytes(8192 + 64) > B.factor_workspace_bytes(8192)
    assert B.factor_workspace_bytes(100) >= 2 * 128 * 128 * 4
    # the one-sided path: working weights and errors, padded copy of P_A when ragged
    assert B.gptq_workspace_bytes(0, 64) == 0
    assert B.gptq_workspace_bytes(128, 128) >= 2 * 128 * 128 * 4
    assert B.gptq_workspace_bytes(100, 70) >= 2 * 128 * 128 * 4 + 128 * 128 * 4


def test_workspace_sizes_at_the_largest_dimension(B):
    # BAKRON_MAX_DIM = 65536: the sizes are computed in 64-bit (a 65536^2 float32 matrix alone is 16 GiB),
    # grow with the problem and cover their lower bounds; one more row or column is refused (0)
    M = 65536
    f32 = 4 * M * M
    assert B.solve_workspace_bytes(M, M) >= 3 * f32
    assert B.solve_workspace_bytes(M, M) > B.solve_workspace_bytes(M - 64, M - 64) > 0
    assert B.factor_workspace_bytes(M) >= 4 * sum((M // 2 >> d) ** 2 for d in range(9))
    assert B.factor_workspace_bytes(M) > B.factor_workspace_bytes(M - 64) > 0
    assert B.quantize_workspace_bytes(M, M) >= (2 * B.factor_workspace_bytes(M) + B.solve_workspace_bytes(M, M))
    assert B.gptq_workspace_bytes(M, M) >= 2 * f32
    assert B.solve_workspace_bytes(M + 1, 64) == 0 and B.factor_workspace_bytes(M + 1) == 0
    assert B.gptq_workspace_bytes(64, M + 1) == 0 and B.quantize_workspace_bytes(M + 1, 64) == 0


def test_host_side_argument_errors(B):
    L = B.lib()
    fake = ctypes.c_void_p(4096)       # never dereferenced: every call below fails its host checks
    # negative / oversized dimensions
    assert L.bakron_factor(fake, -1, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None) == -2
    assert L.bakron_factor(fake, 65537, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None) == -2
    # bad damping
    assert L.bakron_factor(fake, 8, ctypes.c_float(float("nan")), fake, fake, fake, fake, 1 << 30, None) == -4
    assert L.bakron_factor(fake, 8, ctypes.c_float(-1.0), fake, fake, fake, fake, 1 << 30, None) == -4
    # null pointers
    assert L.bakron_factor(None, 8, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None) == -1
    # n == 0 is a no-op success
    assert L.bakron_factor(None, 0, ctypes.c_float(0.01), None, None, None, None, 0, None) == 0
    # workspace too small / misaligned
    assert L.bakron_factor(fake, 8, ctypes.c_float(0.01), fake, fake, fake, fake, 16, None) == -3
    assert L.bakron_factor(fake, 8, ctypes.c_float(0.01), fake, fake, fake, ctypes.c_void_p(4100), 1 << 30, None) == -3
    # misaligned output matrix
    assert L.bakron_factor(fake, 8, ctypes.c_float(0.01), ctypes.c_void_p(4100), fake, fake, fake, 1 << 30, None) == -4
    args = [fake, 64, 64, fake, fake, fake, fake, fake, fake, fake, fake, fake, None, None, fake, 1 << 30, None]
    a = list(args); a[0] = None
    assert L.bakron_solve(*a) == -1
    a = list(args); a[1] = -3
    assert L.bakron_solve(*a) == -2
    a = list(args); a[1] = 0
    assert L.bakron_solve(*a) == 0
    a = list(args); a[13] = fake; a[3] = None      # objective requested without L_A
    assert L.bakron_solve(*a) == -1
    a = list(args); a[15] = 100
    assert L.bakron_solve(*a) == -3
    a = list(args); a[4] = ctypes.c_void_p(4104)   # misaligned P_A
    assert L.bakron_solve(*a) == -4
    # bakron_gptq(W, m, n, L_A, P_A, scale, zero, maxq, V, codes, err, objective, ws, bytes, stream)
    g = [fake, 64, 64, fake, fake, fake, fake, fake, fake, fake, None, None, fake, 1 << 30, None]
    a = list(g); a[4] = None
    assert L.bakron_gptq(*a) == -1
    a = list(g); a[2] = 65537
    assert L.bakron_gptq(*a) == -2
    a = list(g); a[1] = 0
    assert L.bakron_gptq(*a) == 0
    a = list(g); a[11] = fake; a[3] = None          # objective requested without L_A
    assert L.bakron_gptq(*a) == -1
    # bakron_quantize(W, m, n, A, B, damp, scale, zero, maxq, L_A, P_A, info_A, L_B, P_B, info_B,
    #                 V, codes, err, objective, ws, bytes, stream)
    q = [fake, 64, 64, fake, fake, ctypes.c_float(0.01), fake, fake, fake, fake, fake, fake, fake, fake, fake,
         fake, fake, None, None, fake, 1 << 30, None]
    a = list(q); a[4] = None
    assert L.bakron_quantize(*a) == -1
    a = list(q); a[1] = -1
    assert L.bakron_quantize(*a) == -2
    a = list(q); a[5] = ctypes.c_float(-0.5)
    assert L.bakron_quantize(*a) == -4
    a = list(q); a[2] = 0
    assert L.bakron_quantize(*a) == 0
    a = list(q); a[20] = 1000
    assert L.bakron_quantize(*a) == -3
    a = list(q); a[13] = ctypes.c_void_p(4104)      # misaligned P_B
    assert L.bakron_quantize(*a) == -4
    a = list(g); a[13] = 100
    assert L.bakron_gptq(*a) == -3
    a = list(g); a[4] = ctypes.c_void_p(4104)
    assert L.bakron_gptq(*a) == -4
    # bakron_moment(X, N, n, w, scale, M, stream) / bakron_row_sqnorms(X, N, n, out, stream)
    one = ctypes.c_float(1.0)
    assert L.bakron_moment(fake, 16, 6, None, one, fake, None) == -4            # n not a multiple of 4
    assert L.bakron_moment(ctypes.c_void_p(4100), 16, 8, None, one, fake, None) == -4   # misaligned X
    assert L.bakron_moment(fake, -1, 8, None, one, fake, None) == -2
    assert L.bakron_moment(fake, 16, 65540, None, one, fake, None) == -2
    assert L.bakron_moment(None, 16, 8, None, one, fake, None) == -1
    assert L.bakron_moment(fake, 16, 8, None, one, None, None) == -1
    assert L.bakron_moment(fake, 16, 8, None, ctypes.c_float(float("nan")), fake, None) == -4
    assert L.bakron_moment(None, 16, 0, None, one, None, None) == 0
    assert L.bakron_row_sqnorms(fake, 16, 10, fake, None) == -4
    assert L.bakron_row_sqnorms(fake, 16, 8, None, None) == -1
    assert L.bakron_row_sqnorms(None, 0, 0, None, None) == 0
    # batches: every layer is checked before anything is enqueued
    from two_sided_hessian_amd._binding import Layer
    f = 4096
    good = Layer(f, 64, 64, f, f, f, f, f, f, f, f, f, None, None)
    bad = Layer(f, 64, 64, f, None, f, f, f, f, f, f, f, None, None)       # no P_A
    ragged = Layer(f, 100, 70, f, f, f, f, f, f, f, f, f, None, None)
    arr = (Layer * 3)(good, ragged, bad)
    st = (ctypes.c_void_p * 2)(None, None)
    assert L.bakron_solve_batch(arr, 3, fake, 1 << 40, st, 2) == -1
    assert L.bakron_solve_batch(arr, 2, fake, 100, st, 2) == -3
    assert L.bakron_solve_batch(arr, 2, fake, 1 << 40, st, 0) == -4
    assert L.bakron_solve_batch(arr, 0, None, 0, None, 0) == 0
    # bakron_solve_noalloc(W, m, n, L_A, P_A, L_B, P_B, scale, zero, maxq, V, codes, err, objective, stream):
    # the argument checks of bakron_solve, then the size check against its
    # fixed scratch, all before any device call
    na = [fake, 64, 64, fake, fake, fake, fake, fake, fake, fake, fake, fake, None, None, None]
    a = list(na); a[4] = None
    assert L.bakron_solve_noalloc(*a) == -1
    a = list(na); a[2] = -5
    assert L.bakron_solve_noalloc(*a) == -2
    a = list(na); a[1] = 0
    assert L.bakron_solve_noalloc(*a) == 0
    a = list(na); a[13] = fake; a[5] = None         # objective requested without L_B
    assert L.bakron_solve_noalloc(*a) == -1
    a = list(na); a[6] = ctypes.c_void_p(4104)      # misaligned P_B
    assert L.bakron_solve_noalloc(*a) == -4
    a = list(na); a[1], a[2] = 8192, 8192           # 12 m n bytes, far beyond 256 MiB
    assert L.bakron_solve_noalloc(*a) == -6
    a = list(na); a[1], a[2] = 4096, 8192           # 384 MiB
    assert L.bakron_solve_noalloc(*a) == -6
    assert "noalloc" in B.strerror(-6)
    # the unsplit workspace of a 4096 x 4096 layer fits the scratch
    lay = Layer(f, 4096, 4096, f, f, f, f, f, f, f, f, f, None, None)
    assert L.bakron_solve_batch_workspace_bytes((Layer * 1)(lay), 1, 1) <= B._binding.BAKRON_NOALLOC_SCRATCH_BYTES
    # grouped grids: the group size must be a positive multiple of 64
    sg = [fake, 64, 200, fake, fake, fake, fake, fake, fake, fake, 128, fake, fake, None, None, fake, 1 << 30, None]
    for bad in (0, -64, 96, 1):
        a = list(sg); a[10] = bad
        assert L.bakron_solve_grouped(*a) == -4, bad
    a = list(sg); a[0] = None
    assert L.bakron_solve_grouped(*a) == -1
    a = list(sg); a[16] = 100
    assert L.bakron_solve_grouped(*a) == -3
    a = list(sg); a[1] = 0
    assert L.bakron_solve_grouped(*a) == 0
    gg = [fake, 64, 200, fake, fake, fake, fake, fake, 64, fake, fake, None, None, fake, 1 << 30, None]
    a = list(gg); a[8] = 32
    assert L.bakron_gptq_grouped(*a) == -4
    a = list(gg); a[4] = None
    assert L.bakron_gptq_grouped(*a) == -1
    a = list(gg); a[14] = 64
    assert L.bakron_gptq_grouped(*a) == -3
    # one slice per stream, each sized for its largest layer
    one = L.bakron_solve_batch_workspace_bytes(arr, 2, 1)
    two = L.bakron_solve_batch_workspace_bytes(arr, 2, 2)
    assert one == L.bakron_solve_workspace_bytes(100, 70)
    assert two == L.bakron_solve_workspace_bytes(64, 64) + L.bakron_solve_workspace_bytes(100, 70)


def test_profiled_calls_reject_bad_arguments_on_host(B):
    L = B.lib()
    from two_sided_hessian_amd._binding import KernelStat
    arr = (KernelStat * 16)()
    cnt = ctypes.c_int32(-7)
    fake = ctypes.c_void_p(4096)
    rc = L.bakron_factor_profiled(fake, -1, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None,
                                  arr, 16, ctypes.byref(cnt))
    assert rc == -2 and cnt.value == 0
    rc = L.bakron_factor_profiled(fake, 8, ctypes.c_float(0.01), fake, fake, fake, fake, 1 << 30, None,
                                  arr, 16, None)
    assert rc == -1
    args = [None, 64, 64, fake, fake, fake, fake, fake, fake, fake, fake, fake, None, None, fake, 1 << 30, None]
    assert L.bakron_solve_profiled(*args, arr, 16, ctypes.byref(cnt)) == -1
