"""GPU parity of the Kronecker-factor construction (bakron_row_sqnorms,
bakron_moment, through the C ABI) against the float64 oracle.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians", Hessian choices.

Tolerance: a float32 dot product of length N in any summation order is
within gamma = (N + 4) 2^-24 of the exact value relative to the sum of the
magnitudes of its terms (the weights and the scale add two roundings), so
|M_gpu - M| <= gamma * scale * (|X|^T diag|w| |X|) elementwise, and
|sqnorm_gpu - sqnorm| <= (n + 2) 2^-24 sqnorm.
"""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B
import workloads as WL
from oracle import reference as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U32 = 2.0 ** -24


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def check_moment(X, w, M, rows, label, scale=None):
    X64 = X.astype(np.float64)
    N = X.shape[0]
    sc = (1.0 / N) if scale is None else scale
    w64 = None if w is None else w.astype(np.float64)
    Xw = X64 if w64 is None else X64 * w64[:, None]
    aXw = np.abs(Xw)
    aX = np.abs(X64)
    worst = 0.0
    for i in rows:
        ref = sc * (Xw[:, i] @ X64[:, : i + 1])
        bound = (N + 4) * U32 * abs(sc) * (aXw[:, i] @ aX[:, : i + 1]) + 1e-300
        worst = max(worst, float(np.max(np.abs(M[i, : i + 1] - ref) / bound)))
    print(f"{label}: worst error / bound {worst:.3g}", flush=True)
    assert worst <= 1.0


@pytest.mark.parametrize("N,n,weighted,seed", [(64, 64, False, 0), (300, 100, False, 1), (37, 12, True, 2),
                                              (1000, 260, True, 3), (129, 384, False, 4), (5, 8, True, 5)])
def test_moment_matches_oracle(N, n, weighted, seed):
    rng = np.random.default_rng(seed)
    X = (rng.standard_normal((N, n)) * np.exp(rng.standard_normal(n))[None, :]).astype(np.float32)
    w = (rng.random(N) * 3).astype(np.float32) if weighted else None
    sentinel = -7.25
    M = torch.full((n, n), sentinel, dtype=torch.float32, device=DEV)
    B.moment(to_dev(X), None if w is None else to_dev(w), out=M)
    torch.cuda.synchronize()
    M = M.cpu().numpy()
    assert np.all(np.triu(M, 1)[np.triu_indices(n, 1)] == sentinel), "strict upper triangle was written"
    check_moment(X, w, M, range(n), f"moment {N}x{n} weighted={weighted}")


def test_row_sqnorms_match_oracle():
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((333, 68)) * 3).astype(np.float32)
    got = B.row_sqnorms(to_dev(X)).cpu().numpy().astype(np.float64)
    ref = R.row_sqnorms(X)
    assert np.all(np.abs(got - ref) <= (68 + 2) * U32 * ref)


def test_kfac_and_shampoo_factors_small():
    rng = np.random.default_rng(8)
    Xa = rng.standard_normal((200, 48)).astype(np.float32)
    Xb = rng.standard_normal((200, 40)).astype(np.float32)
    A, Bm = (t.cpu().numpy() for t in B.kfac_factors(to_dev(Xa), to_dev(Xb)))
    check_moment(Xa, None, A, range(48), "kfac A")
    check_moment(Xb, None, Bm, range(40), "kfac B")
    A, Bm = (t.cpu().numpy() for t in B.shampoo_factors(to_dev(Xa), to_dev(Xb)))
    wa, wb = R.row_sqnorms(Xa), R.row_sqnorms(Xb)
    # weights from the oracle's norms: the GPU norms differ by rounding,
    # which the bound absorbs (relative (n + 2) 2^-24 per weight)
    Aref, Bref = R.shampoo_factors(Xa, Xb)
    for M, ref, X, w in ((A, Aref, Xa, wb), (Bm, Bref, Xb, wa)):
        aM = np.abs(X.astype(np.float64) * w[:, None]).T @ np.abs(X.astype(np.float64)) / X.shape[0]
        tri = np.tril_indices(M.shape[0])
        err = np.abs(M[tri] - ref[tri]) / ((X.shape[0] + 60) * U32 * aM[tri] + 1e-300)
        assert err.max() <= 1.0, err.max()


def test_moment_edges():
    X = to_dev(np.ones((4, 8), np.float32))
    M = torch.full((8, 8), 3.0, device=DEV)
    lib = B.lib()
    import ctypes
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    # N == 0 writes zeros to the lower triangle
    assert lib.bakron_moment(p(X), 0, 8, None, ctypes.c_float(1.0), p(M), None) == 0
    torch.cuda.synchronize()
    Mh = M.cpu().numpy()
    assert np.all(np.tril(Mh) == 0) and np.all(Mh[np.triu_indices(8, 1)] == 3.0)
    # n not a multiple of 4, n == 0, null output
    assert lib.bakron_moment(p(X), 4, 6, None, ctypes.c_float(1.0), p(M), None) == -4
    assert lib.bakron_moment(None, 4, 0, None, ctypes.c_float(1.0), None, None) == 0
    assert lib.bakron_moment(p(X), 4, 8, None, ctypes.c_float(1.0), None, None) == -1
    assert lib.bakron_moment(p(X), 4, 8, None, ctypes.c_float(float("inf")), p(M), None) == -4


@pytest.mark.parametrize("name", ["sq8192_mixed", "glu_up_4096x14336"])
def test_factors_full_size_sampled_rows(name):
    spec = WL.by_name(name)
    S = WL.samples(spec)
    Xa, Xb = S["X"], S["G"]
    print(f"factors {name}: X {Xa.shape}, G {Xb.shape}", flush=True)
    da, db = to_dev(Xa), to_dev(Xb)
    A, Bm = B.kfac_factors(da, db)
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    for M, X, tag in ((A, Xa, "A"), (Bm, Xb, "B")):
        n = X.shape[1]
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=10, replace=False)]))
        Mh = M[torch.as_tensor(rows, device=DEV)].cpu().numpy()
        full = np.zeros((n, n), np.float32)
        full[rows] = Mh
        check_moment(X, None, full, rows, f"{name} kfac {tag}")
    wb = B.row_sqnorms(db)
    As = B.moment(da, wb)
    torch.cuda.synchronize()
    w = wb.cpu().numpy()
    n = Xa.shape[1]
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, size=8, replace=False)]))
    full = np.zeros((n, n), np.float32)
    full[rows] = As[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    check_moment(Xa, w, full, rows, f"{name} shampoo A")
