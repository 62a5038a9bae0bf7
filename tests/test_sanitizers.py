"""Host-side sanitizer builds, run on the CPU (no GPU, no GPU sanitizer).

* The C oracle (oracle/recursive.c) with AddressSanitizer and
  UndefinedBehaviorSanitizer, driven by tests/sanitize/oracle_check.c over
  ragged shapes, leaf sizes, per-row and per-group grids, tie following and
  the argument errors.
* The library's host code (every csrc/*.hip, sanitizers on the host side
  only) linked with tests/sanitize/abi_check.cpp, which drives the C ABI's
  host paths: workspace sizes over many shapes, every host-side argument
  error, batch descriptor checks, the no-allocation call's size limit.
Any sanitizer report aborts the driver (no recovery), so the test fails.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "two_sided_hessian_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
           OMP_NUM_THREADS="2")


def _run(cmd, cwd, **kw):
    r = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          "-fopenmp", os.path.join(SAN, "oracle_check.c"), os.path.join(ROOT, "oracle", "recursive.c"), "-o", exe,
          "-lm"], str(tmp_path))
    out = _run([exe], str(tmp_path), env=ENV, timeout=600)
    assert "ORACLE SANITIZE OK" in out


@pytest.mark.skipif(not os.path.exists(HIPCC) or not os.path.exists(CLANGXX), reason="ROCm toolchain not found")
def test_c_abi_host_paths_under_asan_ubsan(tmp_path):
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    procs = []
    objs = []
    for f in srcs:
        obj = str(tmp_path / f.replace(".hip", ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen(
            [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, f), "-o", obj],
            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for f, p in zip(srcs, procs):
        out = p.communicate()[0]
        assert p.returncode == 0, f"{f}\n{out[-4000:]}"
    drv = str(tmp_path / "abi_check.o")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-c", os.path.join(SAN, "abi_check.cpp"),
          "-o", drv], str(tmp_path))
    exe = str(tmp_path / "abi_check")
    _run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined", drv] + objs + ["-o", exe],
         str(tmp_path))
    out = _run([exe], str(tmp_path), env=ENV, timeout=300)
    assert "ABI SANITIZE OK" in out
