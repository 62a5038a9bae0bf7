"""ctypes binding of libbakron.so (argument marshalling only).

Names follow include/bakron.h.  Tensors are torch CUDA (HIP) tensors; the
binding allocates outputs and the workspace with torch, passes raw device
pointers and the current stream, and checks the return code.  Every
arithmetic step runs in the library's HIP kernels.  There is no fallback:
if libbakron.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbakron.so")

BAKRON_SUCCESS = 0
BAKRON_ERR_NULL_POINTER = -1
BAKRON_ERR_BAD_SIZE = -2
BAKRON_ERR_WORKSPACE = -3
BAKRON_ERR_BAD_ARG = -4
BAKRON_ERR_HIP = -5
BAKRON_ERR_TOO_LARGE = -6
BAKRON_MAX_DIM = 65536
BAKRON_NOALLOC_SCRATCH_BYTES = 256 << 20

# name -> (restype, argtypes); mirrors include/bakron.h
_VP, _I64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "bakron_version": (ctypes.c_int, []),
    "bakron_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "bakron_factor_workspace_bytes": (_SZ, [_I64]),
    "bakron_factor": (ctypes.c_int, [_VP, _I64, ctypes.c_float, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "bakron_solve_workspace_bytes": (_SZ, [_I64, _I64]),
    "bakron_solve": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                    _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "bakron_solve_grouped": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64,
                                            _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "bakron_gptq_grouped": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP, _VP,
                                           _VP, _SZ, _VP]),
    "bakron_solve_antidiagonal_workspace_bytes": (_SZ, [_I64, _I64]),
    "bakron_solve_antidiagonal": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                                 _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "bakron_gptq_workspace_bytes": (_SZ, [_I64, _I64]),
    "bakron_gptq": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
    "bakron_row_sqnorms": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP]),
    "bakron_moment": (ctypes.c_int, [_VP, _I64, _I64, _VP, ctypes.c_float, _VP, _VP]),
    "bakron_solve_noalloc": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                            _VP, _VP, _VP, _VP, _VP]),
    "bakron_quantize_workspace_bytes": (_SZ, [_I64, _I64]),
    "bakron_quantize": (ctypes.c_int, [_VP, _I64, _I64, _VP, _VP, ctypes.c_float, _VP, _VP, _VP,
                                       _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
}



class Layer(ctypes.Structure):
    """bakron_layer (include/bakron.h)."""
    _fields_ = [("W", _VP), ("m", _I64), ("n", _I64), ("L_A", _VP), ("P_A", _VP), ("L_B", _VP), ("P_B", _VP),
                ("scale", _VP), ("zero", _VP), ("maxq", _VP), ("V", _VP), ("codes", _VP), ("err", _VP),
                ("objective", _VP)]


SIGNATURES["bakron_solve_batch_workspace_bytes"] = (_SZ, [ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_int32])
SIGNATURES["bakron_solve_batch"] = (ctypes.c_int, [ctypes.POINTER(Layer), ctypes.c_int32, _VP, _SZ,
                                                   ctypes.POINTER(_VP), ctypes.c_int32])


class KernelStat(ctypes.Structure):
    """bakron_kernel_stat (include/bakron.h)."""
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double),
                ("alg_flops", ctypes.c_double), ("alg_bytes", ctypes.c_double)]


BAKRON_MAX_KERNEL_KINDS = 48
_PSTAT = ctypes.POINTER(KernelStat)
SIGNATURES["bakron_factor_profiled"] = (ctypes.c_int, SIGNATURES["bakron_factor"][1] + [_PSTAT, ctypes.c_int32, _VP])
SIGNATURES["bakron_solve_profiled"] = (ctypes.c_int, SIGNATURES["bakron_solve"][1] + [_PSTAT, ctypes.c_int32, _VP])
SIGNATURES["bakron_gptq_profiled"] = (ctypes.c_int, SIGNATURES["bakron_gptq"][1] + [_PSTAT, ctypes.c_int32, _VP])
SIGNATURES["bakron_solve_antidiagonal_profiled"] = (ctypes.c_int, SIGNATURES["bakron_solve_antidiagonal"][1] +
                                                   [_PSTAT, ctypes.c_int32, _VP])
SIGNATURES["bakron_moment_profiled"] = (ctypes.c_int, SIGNATURES["bakron_moment"][1] + [_PSTAT, ctypes.c_int32, _VP])

_lib = None


class BakronError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} (code {code})")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libbakron.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "(or python two_sided_hessian_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def strerror(code: int) -> str:
    return lib().bakron_strerror(int(code)).decode()


def version() -> int:
    return lib().bakron_version()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, dtype, shape):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class GridError(ValueError):
    """A per-row grid that breaks the contract of include/bakron.h."""


MAXQ_LIMIT = 255   # codes are stored as uint8


def check_grid(scale, zero, maxq) -> None:
    """Raise GridError unless every scale is finite and > 0, every zero point
    finite and every maxq in [1, 255] (the grid contract of bakron_solve,
    bakron_quantize and bakron_gptq; the device does not check it).  Takes
    torch tensors on any device (a device tensor is copied to the host, which
    waits for the work that produces it) or numpy arrays."""
    def host(x):
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu")
        return torch.as_tensor(x)
    s, z, q = host(scale), host(zero), host(maxq)
    if s.numel() and not bool(torch.isfinite(s).all()):
        raise GridError("scale must be finite")
    if s.numel() and not bool((s > 0).all()):
        raise GridError("scale must be > 0")
    if z.numel() and not bool(torch.isfinite(z).all()):
        raise GridError("zero must be finite")
    if q.numel() and not bool(((q >= 1) & (q <= MAXQ_LIMIT)).all()):
        raise GridError(f"maxq must lie in [1, {MAXQ_LIMIT}]")


def workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns >= 512-byte aligned blocks
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def factor_workspace_bytes(n: int) -> int:
    return lib().bakron_factor_workspace_bytes(int(n))


def solve_workspace_bytes(m: int, n: int) -> int:
    return lib().bakron_solve_workspace_bytes(int(m), int(n))


def gptq_workspace_bytes(m: int, n: int) -> int:
    return lib().bakron_gptq_workspace_bytes(int(m), int(n))


def _stats_out():
    arr = (KernelStat * BAKRON_MAX_KERNEL_KINDS)()
    cnt = ctypes.c_int32(0)
    return arr, cnt


def _stats_list(arr, cnt):
    return [{"name": arr[i].name.decode(), "launches": arr[i].launches, "total_ms": arr[i].total_ms,
             "alg_flops": arr[i].alg_flops, "alg_bytes": arr[i].alg_bytes} for i in range(cnt.value)]


def factor(A: torch.Tensor, damp_frac: float = 0.01, *, out=None, ws=None, stream=None, profile=None):
    """bakron_factor: returns (L, P, info) device tensors; info is int32[1]
    (0 = success), valid once the stream has been synchronised.  With a list
    passed as ``profile``, runs bakron_factor_profiled (synchronises) and
    appends its per-kernel statistics to the list."""
    n = A.shape[0]
    _check_dev("A", A, torch.float32, (n, n))
    dev = A.device
    if out is None:
        L = torch.empty((n, n), dtype=torch.float32, device=dev)
        P = torch.empty((n, n), dtype=torch.float32, device=dev)
        info = torch.empty((1,), dtype=torch.int32, device=dev)
    else:
        L, P, info = out
    need = factor_workspace_bytes(n)
    if ws is None:
        ws = workspace(need, dev)
    args = [_ptr(A), n, ctypes.c_float(damp_frac), _ptr(L), _ptr(P), _ptr(info), _ptr(ws), ws.numel(),
            _stream(stream)]
    if profile is None:
        rc = lib().bakron_factor(*args)
    else:
        arr, cnt = _stats_out()
        rc = lib().bakron_factor_profiled(*args, arr, BAKRON_MAX_KERNEL_KINDS, ctypes.byref(cnt))
        profile.extend(_stats_list(arr, cnt))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_factor")
    return L, P, info


def _grid_shape(m, n, group_size):
    if group_size is None:
        return (m,)
    if group_size <= 0 or group_size % 64:
        raise ValueError("group_size must be a positive multiple of 64")
    return (m, -(-n // group_size))


def solve(W, LA, PA, LB, PB, scale, zero, maxq, *, want_err=False, want_objective=True,
          out=None, ws=None, stream=None, profile=None, check=True, group_size=None):
    """bakron_solve: returns dict(V, codes, err?, objective?) of device tensors.
    ``profile``: as in factor().  ``check``: check the grid contract first
    (check_grid; it reads the grid back to the host, so a caller that runs
    the same grid many times may check it once and pass check=False).
    ``group_size``: per-group grids (bakron_solve_grouped; scale, zero, maxq
    m x ceil(n / group_size))."""
    m, n = W.shape
    gshape = _grid_shape(m, n, group_size)
    _check_dev("W", W, torch.float32, (m, n))
    _check_dev("P_A", PA, torch.float32, (n, n))
    _check_dev("P_B", PB, torch.float32, (m, m))
    _check_dev("scale", scale, torch.float32, gshape)
    _check_dev("zero", zero, torch.float32, gshape)
    _check_dev("maxq", maxq, torch.int32, gshape)
    if group_size is not None and profile is not None:
        raise ValueError("the profiled solve takes per-row grids only")
    if want_objective:
        _check_dev("L_A", LA, torch.float32, (n, n))
        _check_dev("L_B", LB, torch.float32, (m, m))
    if check:
        check_grid(scale, zero, maxq)
    dev = W.device
    if out is None:
        out = {
            "V": torch.empty((m, n), dtype=torch.float32, device=dev),
            "codes": torch.empty((m, n), dtype=torch.uint8, device=dev),
        }
        if want_err:
            out["err"] = torch.empty((m, n), dtype=torch.float32, device=dev)
        if want_objective:
            out["objective"] = torch.empty((1,), dtype=torch.float64, device=dev)
    need = solve_workspace_bytes(m, n)
    if ws is None:
        ws = workspace(need, dev)
    args = [_ptr(W), m, n, _ptr(LA) if want_objective else None, _ptr(PA),
            _ptr(LB) if want_objective else None, _ptr(PB), _ptr(scale), _ptr(zero),
            _ptr(maxq), _ptr(out["V"]), _ptr(out["codes"]), _ptr(out.get("err")),
            _ptr(out.get("objective")), _ptr(ws), ws.numel(), _stream(stream)]
    if group_size is not None:
        rc = lib().bakron_solve_grouped(*(args[:10] + [int(group_size)] + args[10:]))
        if rc != BAKRON_SUCCESS:
            raise BakronError(rc, "bakron_solve_grouped")
        return out
    if profile is None:
        rc = lib().bakron_solve(*args)
    else:
        arr, cnt = _stats_out()
        rc = lib().bakron_solve_profiled(*args, arr, BAKRON_MAX_KERNEL_KINDS, ctypes.byref(cnt))
        profile.extend(_stats_list(arr, cnt))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_solve")
    return out


def solve_noalloc(W, LA, PA, LB, PB, scale, zero, maxq, *, want_err=False, want_objective=True, out=None,
                  stream=None, check=True):
    """bakron_solve_noalloc (no workspace: the library's fixed device scratch;
    the results are bakron_solve's).  Returns dict(V, codes, err?,
    objective?).  With ``out`` given and check=False it allocates nothing and
    only enqueues kernels, so it can be captured into a HIP graph (make one
    call before capturing: the first call on a device looks the scratch up).
    ``check``: as in solve(); it reads the grid back to the host, which
    graph capture does not allow."""
    m, n = W.shape
    _check_dev("W", W, torch.float32, (m, n))
    _check_dev("P_A", PA, torch.float32, (n, n))
    _check_dev("P_B", PB, torch.float32, (m, m))
    _check_dev("scale", scale, torch.float32, (m,))
    _check_dev("zero", zero, torch.float32, (m,))
    _check_dev("maxq", maxq, torch.int32, (m,))
    if want_objective:
        _check_dev("L_A", LA, torch.float32, (n, n))
        _check_dev("L_B", LB, torch.float32, (m, m))
    if check:
        check_grid(scale, zero, maxq)
    dev = W.device
    if out is None:
        out = {"V": torch.empty((m, n), dtype=torch.float32, device=dev),
               "codes": torch.empty((m, n), dtype=torch.uint8, device=dev)}
        if want_err:
            out["err"] = torch.empty((m, n), dtype=torch.float32, device=dev)
        if want_objective:
            out["objective"] = torch.empty((1,), dtype=torch.float64, device=dev)
    rc = lib().bakron_solve_noalloc(_ptr(W), m, n, _ptr(LA) if want_objective else None, _ptr(PA),
                                    _ptr(LB) if want_objective else None, _ptr(PB), _ptr(scale), _ptr(zero),
                                    _ptr(maxq), _ptr(out["V"]), _ptr(out["codes"]), _ptr(out.get("err")),
                                    _ptr(out.get("objective")), _stream(stream))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_solve_noalloc")
    return out


def solve_antidiagonal(W, LA, PA, LB, PB, scale, zero, maxq, *, want_err=False, want_objective=True, out=None,
                       ws=None, stream=None, profile=None, check=True):
    """bakron_solve_antidiagonal (one entry anti-diagonal per step): returns
    dict(V, codes, err?, objective?) of device tensors.  ``profile``: as in
    factor(); ``check``: as in solve()."""
    m, n = W.shape
    _check_dev("W", W, torch.float32, (m, n))
    _check_dev("P_A", PA, torch.float32, (n, n))
    _check_dev("P_B", PB, torch.float32, (m, m))
    _check_dev("scale", scale, torch.float32, (m,))
    _check_dev("zero", zero, torch.float32, (m,))
    _check_dev("maxq", maxq, torch.int32, (m,))
    if want_objective:
        _check_dev("L_A", LA, torch.float32, (n, n))
        _check_dev("L_B", LB, torch.float32, (m, m))
    if check:
        check_grid(scale, zero, maxq)
    dev = W.device
    if out is None:
        out = {"V": torch.empty((m, n), dtype=torch.float32, device=dev),
               "codes": torch.empty((m, n), dtype=torch.uint8, device=dev)}
        if want_err:
            out["err"] = torch.empty((m, n), dtype=torch.float32, device=dev)
        if want_objective:
            out["objective"] = torch.empty((1,), dtype=torch.float64, device=dev)
    if ws is None:
        ws = workspace(lib().bakron_solve_antidiagonal_workspace_bytes(m, n), dev)
    args = [_ptr(W), m, n, _ptr(LA) if want_objective else None, _ptr(PA), _ptr(LB) if want_objective else None,
            _ptr(PB), _ptr(scale), _ptr(zero), _ptr(maxq), _ptr(out["V"]), _ptr(out["codes"]), _ptr(out.get("err")),
            _ptr(out.get("objective")), _ptr(ws), ws.numel(), _stream(stream)]
    if profile is None:
        rc = lib().bakron_solve_antidiagonal(*args)
    else:
        arr, cnt = _stats_out()
        rc = lib().bakron_solve_antidiagonal_profiled(*args, arr, BAKRON_MAX_KERNEL_KINDS, ctypes.byref(cnt))
        profile.extend(_stats_list(arr, cnt))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_solve_antidiagonal")
    return out


def quantize_workspace_bytes(m: int, n: int) -> int:
    return int(lib().bakron_quantize_workspace_bytes(m, n))


def quantize(W, A, B, scale, zero, maxq, damp_frac: float = 0.01, *, want_err=False, want_objective=True,
             out=None, ws=None, stream=None, check=True):
    """bakron_quantize (both factors and the solve in one call): returns
    dict(V, codes, err?, objective?, L_A, P_A, info_A, L_B, P_B, info_B) of
    device tensors.  ``check``: as in solve()."""
    m, n = W.shape
    _check_dev("W", W, torch.float32, (m, n))
    _check_dev("A", A, torch.float32, (n, n))
    _check_dev("B", B, torch.float32, (m, m))
    _check_dev("scale", scale, torch.float32, (m,))
    _check_dev("zero", zero, torch.float32, (m,))
    _check_dev("maxq", maxq, torch.int32, (m,))
    if check:
        check_grid(scale, zero, maxq)
    dev = W.device
    if out is None:
        out = {
            "V": torch.empty((m, n), dtype=torch.float32, device=dev),
            "codes": torch.empty((m, n), dtype=torch.uint8, device=dev),
            "L_A": torch.empty((n, n), dtype=torch.float32, device=dev),
            "P_A": torch.empty((n, n), dtype=torch.float32, device=dev),
            "info_A": torch.zeros((1,), dtype=torch.int32, device=dev),
            "L_B": torch.empty((m, m), dtype=torch.float32, device=dev),
            "P_B": torch.empty((m, m), dtype=torch.float32, device=dev),
            "info_B": torch.zeros((1,), dtype=torch.int32, device=dev),
        }
        if want_err:
            out["err"] = torch.empty((m, n), dtype=torch.float32, device=dev)
        if want_objective:
            out["objective"] = torch.empty((1,), dtype=torch.float64, device=dev)
    need = quantize_workspace_bytes(m, n)
    if ws is None:
        ws = workspace(need, dev)
    rc = lib().bakron_quantize(_ptr(W), m, n, _ptr(A), _ptr(B), float(damp_frac), _ptr(scale), _ptr(zero),
                               _ptr(maxq), _ptr(out["L_A"]), _ptr(out["P_A"]), _ptr(out["info_A"]),
                               _ptr(out["L_B"]), _ptr(out["P_B"]), _ptr(out["info_B"]), _ptr(out["V"]),
                               _ptr(out["codes"]), _ptr(out.get("err")), _ptr(out.get("objective")), _ptr(ws),
                               ws.numel(), _stream(stream))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_quantize")
    return out


def gptq(W, LA, PA, scale, zero, maxq, *, want_err=False, want_objective=True, out=None, ws=None, stream=None,
         profile=None, check=True, group_size=None):
    """bakron_gptq (the one-sided case B = I): returns dict(V, codes, err?,
    objective?) of device tensors.  ``profile``: as in factor(); ``check``
    and ``group_size`` (bakron_gptq_grouped): as in solve()."""
    m, n = W.shape
    gshape = _grid_shape(m, n, group_size)
    _check_dev("W", W, torch.float32, (m, n))
    _check_dev("P_A", PA, torch.float32, (n, n))
    _check_dev("scale", scale, torch.float32, gshape)
    _check_dev("zero", zero, torch.float32, gshape)
    _check_dev("maxq", maxq, torch.int32, gshape)
    if group_size is not None and profile is not None:
        raise ValueError("the profiled one-sided call takes per-row grids only")
    if want_objective:
        _check_dev("L_A", LA, torch.float32, (n, n))
    if check:
        check_grid(scale, zero, maxq)
    dev = W.device
    if out is None:
        out = {
            "V": torch.empty((m, n), dtype=torch.float32, device=dev),
            "codes": torch.empty((m, n), dtype=torch.uint8, device=dev),
        }
        if want_err:
            out["err"] = torch.empty((m, n), dtype=torch.float32, device=dev)
        if want_objective:
            out["objective"] = torch.empty((1,), dtype=torch.float64, device=dev)
    need = gptq_workspace_bytes(m, n)
    if ws is None:
        ws = workspace(need, dev)
    args = [_ptr(W), m, n, _ptr(LA) if want_objective else None, _ptr(PA), _ptr(scale), _ptr(zero), _ptr(maxq),
            _ptr(out["V"]), _ptr(out["codes"]), _ptr(out.get("err")), _ptr(out.get("objective")), _ptr(ws),
            ws.numel(), _stream(stream)]
    if group_size is not None:
        rc = lib().bakron_gptq_grouped(*(args[:8] + [int(group_size)] + args[8:]))
        if rc != BAKRON_SUCCESS:
            raise BakronError(rc, "bakron_gptq_grouped")
        return out
    if profile is None:
        rc = lib().bakron_gptq(*args)
    else:
        arr, cnt = _stats_out()
        rc = lib().bakron_gptq_profiled(*args, arr, BAKRON_MAX_KERNEL_KINDS, ctypes.byref(cnt))
        profile.extend(_stats_list(arr, cnt))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_gptq")
    return out


def row_sqnorms(X, *, out=None, stream=None):
    """bakron_row_sqnorms: out[t] = |X[t, :]|^2 (device float32, N)."""
    N, n = X.shape
    _check_dev("X", X, torch.float32, (N, n))
    if out is None:
        out = torch.empty((N,), dtype=torch.float32, device=X.device)
    rc = lib().bakron_row_sqnorms(_ptr(X), N, n, _ptr(out), _stream(stream))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_row_sqnorms")
    return out


def moment(X, w=None, scale=None, *, out=None, stream=None, profile=None):
    """bakron_moment: M = scale * sum_t w_t x_t x_t^T (lower triangle and
    diagonal written; scale defaults to 1 / N).  ``profile``: as in factor()."""
    N, n = X.shape
    _check_dev("X", X, torch.float32, (N, n))
    if w is not None:
        _check_dev("w", w, torch.float32, (N,))
    if scale is None:
        scale = 1.0 / N if N else 0.0
    if out is None:
        out = torch.zeros((n, n), dtype=torch.float32, device=X.device)
    args = [_ptr(X), N, n, _ptr(w), ctypes.c_float(scale), _ptr(out), _stream(stream)]
    if profile is None:
        rc = lib().bakron_moment(*args)
    else:
        arr, cnt = _stats_out()
        rc = lib().bakron_moment_profiled(*args, arr, BAKRON_MAX_KERNEL_KINDS, ctypes.byref(cnt))
        profile.extend(_stats_list(arr, cnt))
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_moment")
    return out


def kfac_factors(Xa, Xb, *, stream=None):
    """K-FAC-style factors from sample-major activations Xa (N x n) and
    output gradients Xb (N x m): A = E[a a^T], B = E[b b^T] (lower
    triangles)."""
    return moment(Xa, stream=stream), moment(Xb, stream=stream)


def shampoo_factors(Xa, Xb, *, stream=None):
    """Shampoo-style factors after one power-iteration step from the
    identity: A = E[|b|^2 a a^T], B = E[|a|^2 b b^T] (lower triangles)."""
    wa, wb = row_sqnorms(Xa, stream=stream), row_sqnorms(Xb, stream=stream)
    return moment(Xa, wb, stream=stream), moment(Xb, wa, stream=stream)


def solve_batch(problems, streams=None, *, want_err=False, want_objective=True, ws=None, check=True):
    """bakron_solve_batch: ``problems`` is a list of dicts with device
    tensors W, LA, PA, LB, PB, scale, zero, maxq (one per layer); layer k runs
    on streams[k % len(streams)] (default: the current stream only).
    Returns one output dict per layer, as solve() does.

    Stream order: the outputs and the workspace are allocated on the current
    stream, so every batch stream first waits for the current stream (the
    inputs may still be in production there), and the current stream waits
    for every batch stream after the call: the outputs are complete for
    later work on the current stream, and the workspace is not handed out
    again by torch's allocator while a batch kernel may still use it.
    ``check``: as in solve(), for every layer."""
    cur = torch.cuda.current_stream()
    if streams is None:
        streams = [cur]
    outs, descs = [], []
    for p in problems:
        W = p["W"]
        m, n = W.shape
        _check_dev("W", W, torch.float32, (m, n))
        _check_dev("P_A", p["PA"], torch.float32, (n, n))
        _check_dev("P_B", p["PB"], torch.float32, (m, m))
        _check_dev("scale", p["scale"], torch.float32, (m,))
        _check_dev("zero", p["zero"], torch.float32, (m,))
        _check_dev("maxq", p["maxq"], torch.int32, (m,))
        if want_objective:
            _check_dev("L_A", p["LA"], torch.float32, (n, n))
            _check_dev("L_B", p["LB"], torch.float32, (m, m))
        if check:
            check_grid(p["scale"], p["zero"], p["maxq"])
        dev = W.device
        o = {"V": torch.empty((m, n), dtype=torch.float32, device=dev),
             "codes": torch.empty((m, n), dtype=torch.uint8, device=dev)}
        if want_err:
            o["err"] = torch.empty((m, n), dtype=torch.float32, device=dev)
        if want_objective:
            o["objective"] = torch.empty((1,), dtype=torch.float64, device=dev)
        outs.append(o)
        descs.append(Layer(W.data_ptr(), m, n, p["LA"].data_ptr() if want_objective else None, p["PA"].data_ptr(),
                           p["LB"].data_ptr() if want_objective else None, p["PB"].data_ptr(),
                           p["scale"].data_ptr(), p["zero"].data_ptr(), p["maxq"].data_ptr(), o["V"].data_ptr(),
                           o["codes"].data_ptr(), o["err"].data_ptr() if want_err else None,
                           o["objective"].data_ptr() if want_objective else None))
    arr = (Layer * max(1, len(descs)))(*descs)
    sarr = (_VP * len(streams))(*[s.cuda_stream for s in streams])
    need = lib().bakron_solve_batch_workspace_bytes(arr, len(descs), len(streams))
    if ws is None:
        ws = workspace(need, problems[0]["W"].device if problems else "cuda")
    for s in streams:
        if s != cur:
            s.wait_stream(cur)
    rc = lib().bakron_solve_batch(arr, len(descs), _ptr(ws), ws.numel(), sarr, len(streams))
    for s in streams:
        if s != cur:
            cur.wait_stream(s)
    if rc != BAKRON_SUCCESS:
        raise BakronError(rc, "bakron_solve_batch")
    return outs
