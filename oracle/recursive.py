"""ctypes front end of ``recursive.c`` (TEST INFRASTRUCTURE ONLY).

Sequential float64 BaKron-recursive (quadtree divide and conquer with naive
leaves), for shapes too large for the numpy forms in ``reference``.  See the
header of ``recursive.c`` for the algorithm and the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "recursive.c")
_LIB = os.path.join(_HERE, "liboracle_recursive.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile recursive.c with gcc (float64, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-march=x86-64-v2", "-fopenmp", "-ffp-contract=off",
                               "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_bakron_recursive
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 6 + \
                     [ctypes.c_int64] + [ctypes.c_void_p] * 3
        g = lib.oracle_bakron_recursive_follow
        g.restype = ctypes.c_int
        g.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 6 + \
                     [ctypes.c_int64] + [ctypes.c_void_p] * 4 + [ctypes.c_double, ctypes.c_void_p]
        h = lib.oracle_bakron_recursive_grouped
        h.restype = ctypes.c_int
        h.argtypes = [ctypes.c_int64, ctypes.c_int64] + [ctypes.c_void_p] * 6 + \
                     [ctypes.c_int64] * 3 + [ctypes.c_void_p] * 4 + [ctypes.c_double, ctypes.c_void_p]
        _lib = lib
    return _lib


def bakron_recursive(W, PA, PB, s, z, maxq, leaf: int = 32, threads: int | None = None, follow=None,
                     tau: float = 1e-4, group_size: int | None = None):
    """Returns (codes int32, V float64, E float64), all m x n.

    With ``follow`` (m x n codes of another implementation) the oracle runs in
    tie-following mode (see recursive.c) and returns (codes, V, E, adoptions).
    Grids are per row (length m), or with ``group_size`` g per (row, group of
    g columns), m x ceil(n / g)."""
    lib = _load()
    W = np.ascontiguousarray(W, dtype=np.float64)
    PA = np.ascontiguousarray(PA, dtype=np.float64)
    PB = np.ascontiguousarray(PB, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float32)
    z = np.ascontiguousarray(z, dtype=np.float32)
    maxq = np.ascontiguousarray(maxq, dtype=np.int32)
    m, n = W.shape
    if group_size is None:
        gshape, group, gld = (m,), max(n, 1), 1
    else:
        group = int(group_size)
        gld = -(-n // group)
        gshape = (m, gld)
    if PA.shape != (n, n) or PB.shape != (m, m) or s.shape != gshape or z.shape != gshape or maxq.shape != gshape:
        raise ValueError("shape mismatch")
    codes = np.zeros((m, n), dtype=np.int32)
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    if threads is not None:
        os.environ["OMP_NUM_THREADS"] = str(int(threads))
    fol = None
    if follow is not None:
        fol = np.ascontiguousarray(follow, dtype=np.int32)
        if fol.shape != (m, n):
            raise ValueError("follow must be m x n")
    adopt = ctypes.c_int64(0)
    rc = lib.oracle_bakron_recursive_grouped(m, n, W.ctypes.data, PA.ctypes.data, PB.ctypes.data,
                                             s.ctypes.data, z.ctypes.data, maxq.ctypes.data, group, gld, int(leaf),
                                             codes.ctypes.data, V.ctypes.data, E.ctypes.data,
                                             None if fol is None else fol.ctypes.data, float(tau),
                                             ctypes.byref(adopt))
    if rc != 0:
        raise RuntimeError("oracle_bakron_recursive_grouped failed with %d" % rc)
    if follow is None:
        return codes, V, E
    return codes, V, E, int(adopt.value)
