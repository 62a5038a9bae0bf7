"""GPU parity of BaKron-antidiagonal (bakron_solve_antidiagonal, through the C
ABI) against the float64 oracle.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (derivation, second variant: BaKron-antidiagonal;
Theorem 3.2: it gives the same rounding as BaKron-naive and BaKron).

The bar is the solve's: the oracle on the same factors (the float64 quadtree
recursion, a different order that Theorem 3.2 makes equivalent), following
the GPU's code only where its own decision lies within TAU grid steps of a
rounding boundary, gives every code equal with at most 1e-4 of the entries
followed; the validator finds no mismatch outside that band; V is s (c - z)
bit for bit; raw errors within 1e-3 grid steps; objective within 1e-3.  The
numpy form of the same algorithm (oracle.reference.bakron_antidiagonal)
gives the same codes on the small shapes away from near-ties.
"""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B
import workloads as WL
from oracle import recursive as O2
from oracle import reference as R
from workloads import make_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TAU = 1e-4


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _check(d, LA, PA, LB, PB, out, label):
    m, n = d["W"].shape
    s, z, mq = d["scale"], d["zero"], d["maxq"]
    codes = out["codes"].astype(np.int64)
    assert np.array_equal(out["V"], (s[:, None] * (codes.astype(np.float32) - z[:, None])).astype(np.float32))
    PA64, PB64 = PA.astype(np.float64), PB.astype(np.float64)
    v = R.validate(d["W"], codes, s, z, mq, tau=TAU, PA=PA64, PB=PB64, return_errors=True)
    E, ties = v.pop("E"), v.pop("tie_mask")
    v.pop("bad_mask")
    c_or, _, E_or, adopted = O2.bakron_recursive(d["W"], PA64, PB64, s, z, mq, follow=codes, tau=TAU)
    diff = int((codes != c_or).sum())
    print(f"{label}: {m}x{n} validator {v}, oracle adopted {adopted}, {diff} differ", flush=True)
    assert v["bad"] == 0 and v["max_step"] <= 1 and v["mismatches"] <= max(1, 1e-4 * m * n)
    assert adopted <= max(1, 1e-4 * m * n) and diff == 0
    assert (np.abs(out["err"] - E) / s[:, None]).max() < 1e-3
    dA, dB = np.diag(LA).astype(np.float64), np.diag(LB).astype(np.float64)
    assert out["objective"][0] == pytest.approx(float(np.sum((dB[:, None] * out["err"] * dA[None, :]) ** 2)),
                                                rel=1e-6)
    assert out["objective"][0] == pytest.approx(float(np.sum((dB[:, None] * E_or * dA[None, :]) ** 2)), rel=1e-3)
    return ties


def _run(d, LA, PA, LB, PB):
    out = B.solve_antidiagonal(to_dev(d["W"]), to_dev(LA), to_dev(PA), to_dev(LB), to_dev(PB), to_dev(d["scale"]),
                               to_dev(d["zero"]), to_dev(d["maxq"]), want_err=True)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("m,n,seed", [(64, 64, 0), (128, 192, 1), (192, 128, 2), (130, 70, 3), (1, 64, 4),
                                      (64, 1, 5), (7, 300, 6), (300, 7, 7), (65, 65, 8), (320, 448, 9),
                                      (200, 136, 10)])
def test_antidiagonal_matches_oracle(m, n, seed):
    d = make_problem(m, n, 500 + seed, global_grid=(n == 1))
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    LB, PB = fb["L"].astype(np.float32), fb["P"].astype(np.float32)
    out = _run(d, LA, PA, LB, PB)
    ties = _check(d, LA, PA, LB, PB, out, "antidiagonal")
    if m * n <= 64 * 64:
        c_np = R.bakron_antidiagonal(d["W"], PA.astype(np.float64), PB.astype(np.float64), d["scale"], d["zero"],
                                     d["maxq"])[0]
        outside = ~R.dependency_cone(ties)
        assert np.array_equal(out["codes"][outside], c_np[outside])


def test_antidiagonal_agrees_with_the_solve():
    # Theorem 3.2 on the GPU: the two algorithms part only inside the
    # dependency cones of near-ties
    d = make_problem(256, 384, 77)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    T = [to_dev(x.astype(np.float32)) for x in (fa["L"], fa["P"], fb["L"], fb["P"])]
    g = [to_dev(d[k]) for k in ("scale", "zero", "maxq")]
    a = B.solve_antidiagonal(to_dev(d["W"]), *T, *g)
    b = B.solve(to_dev(d["W"]), *T, *g)
    torch.cuda.synchronize()
    ca, cb = a["codes"].cpu().numpy(), b["codes"].cpu().numpy()
    ties = np.zeros(ca.shape, bool)
    for c in (ca, cb):
        v = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], tau=TAU, PA=fa["P"], PB=fb["P"],
                       return_errors=True)
        assert v["bad"] == 0
        ties |= v["tie_mask"]
    outside = ~R.dependency_cone(ties)
    assert np.array_equal(ca[outside], cb[outside])
    assert float(a["objective"].item()) == pytest.approx(float(b["objective"].item()), rel=1e-3)


def test_antidiagonal_sq1024_config():
    spec = WL.by_name("sq1024")
    d = WL.generate(spec)
    LA, PA, ia = B.factor(to_dev(d["A"]), 0.01)
    LB, PB, ib = B.factor(to_dev(d["B"]), 0.01)
    torch.cuda.synchronize()
    assert int(ia.item()) == 0 and int(ib.item()) == 0
    LA, PA, LB, PB = (x.cpu().numpy() for x in (LA, PA, LB, PB))
    out = _run(d, LA, PA, LB, PB)
    _check(d, LA, PA, LB, PB, out, "antidiagonal sq1024")
