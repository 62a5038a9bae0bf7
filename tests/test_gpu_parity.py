"""GPU parity of libbakron (through the C ABI) against the float64 oracle.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (derivation, Theorem 3.2, Corollary 3.4).

Tolerances (floating point decides integer codes, so several outputs can be
correct near a rounding boundary):
* codes: at most 1e-4 of the entries may differ from the correct rounding of
  the value they were rounded from, never by more than one step, and only
  within TAU grid steps of a rounding boundary (oracle.reference.validate);
* objective ||L_B (V - W) L_A^T||_F^2 within 1e-3 relative;
* factor: backward error ||L^T L - A_d||_F / ||A_d||_F <= 10 n 2^-24.
"""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B
from oracle import recursive as O2
from oracle import reference as R
from workloads import make_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TAU = 1e-4
U32 = 2.0 ** -24


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_factor(A32, damp=0.01):
    L, P, info = B.factor(to_dev(A32), damp)
    torch.cuda.synchronize()
    return L.cpu().numpy(), P.cpu().numpy(), int(info.item())


def gpu_solve(d, LA, PA, LB, PB):
    out = B.solve(to_dev(d["W"]), to_dev(LA), to_dev(PA), to_dev(LB), to_dev(PB), to_dev(d["scale"]),
                  to_dev(d["zero"]), to_dev(d["maxq"]), want_err=True)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def _problem(m, n, seed, **kw):
    if m * n == 1:
        # a single weight has no range: give it a grid by hand
        d = make_problem(2, 2, seed, **kw)
        d["W"] = d["W"][:1, :1].copy()
        d["A"], d["B"] = d["A"][:1, :1].copy(), d["B"][:1, :1].copy()
        d["scale"] = np.array([0.01], np.float32)
        d["zero"] = np.array([3.3], np.float32)
        d["maxq"] = d["maxq"][:1].copy()
        return d
    return make_problem(m, n, seed, global_grid=(n == 1), **kw)


# --------------------------------------------------------------- factor

@pytest.mark.parametrize("n", [1, 63, 64, 65, 100, 128, 192, 320, 1024])
def test_factor_matches_oracle(n):
    d = _problem(8, n, 3)
    A32 = d["A"]
    L, P, info = gpu_factor(A32)
    assert info == 0
    f = R.factor(A32)
    Ad = f["Ad"]
    print(f"factor n={n}", flush=True)
    assert np.array_equal(np.triu(L, 1), np.zeros_like(L))
    assert np.array_equal(np.triu(P, 1), np.zeros_like(P))
    assert np.all(np.diag(L) > 0)
    np.testing.assert_allclose(np.diag(P), 1.0, rtol=0, atol=4 * U32)
    L64, P64 = L.astype(np.float64), P.astype(np.float64)
    back = np.linalg.norm(L64.T @ L64 - Ad) / np.linalg.norm(Ad)
    assert back <= 10 * n * U32, back
    condL = np.linalg.cond(f["L"])
    inv = np.linalg.norm(L64 @ (P64 / np.diag(L64)[None, :]) - np.eye(n)) / np.sqrt(n)
    assert inv <= 10 * n * U32 * condL, (inv, condL)
    fwd = np.linalg.norm(P64 - f["P"]) / np.linalg.norm(f["P"])
    assert fwd <= 10 * n * U32 * np.linalg.cond(Ad), (fwd, np.linalg.cond(Ad))


def test_factor_reports_nonpositive_pivot():
    n = 128
    A = np.eye(n, dtype=np.float32)
    A[10, 10] = -1.0            # row 10 is the first non-positive pivot met from the bottom up
    _, _, info = gpu_factor(A, 0.0)
    assert info == 11
    _, _, info = gpu_factor(-np.eye(64, dtype=np.float32), 0.0)
    assert info == 64
    A = np.eye(n, dtype=np.float32)
    A[70, 70] = np.nan
    _, _, info = gpu_factor(A, 0.0)
    assert info == 71
    # with damping the NaN reaches every pivot through mean(diag A): the
    # first pivot met (the last row) is reported
    _, _, info = gpu_factor(A, 0.01)
    assert info == n


def test_factor_damping_reading():
    A = np.diag(np.array([1.0, 3.0] * 32, dtype=np.float32))
    L, P, info = gpu_factor(A, 0.01)
    assert info == 0
    np.testing.assert_allclose(np.diag(L) ** 2, np.diag(A) + 0.02, rtol=1e-6)


# ----------------------------------------------------- solve (isolated)

def _check_solve(d, LA, PA, LB, PB, out, label):
    """Compare a GPU solve that used factors (LA, PA, LB, PB) with the oracle
    run on the same factor values (promoted to float64)."""
    m, n = d["W"].shape
    s, z, mq = d["scale"], d["zero"], d["maxq"]
    PA64, PB64 = PA.astype(np.float64), PB.astype(np.float64)
    codes = out["codes"].astype(np.int64)
    # V is the grid value of the code, in float32 as the kernel forms it
    Vexp = s[:, None] * (codes.astype(np.float32) - z[:, None])
    assert np.array_equal(out["V"], Vexp.astype(np.float32)), label
    assert np.all(codes <= mq[:, None])
    v = R.validate(d["W"], codes, s, z, mq, tau=TAU, PA=PA64, PB=PB64, return_errors=True)
    ties = v.pop("tie_mask")
    v.pop("bad_mask"), v.pop("E")
    # the oracle on the same factors, following the GPU's code where its own
    # decision lies within TAU of a rounding boundary (there both roundings
    # are valid and the trajectories would part): every other code is equal
    c_or, V_or, E_or, adopted = O2.bakron_recursive(d["W"], PA64, PB64, s, z, mq, follow=codes, tau=TAU)
    diff = int((codes != c_or).sum())
    print(f"{label}: {m}x{n} validator {v}, oracle adopted {adopted}, differing from it {diff}", flush=True)
    assert v["bad"] == 0 and v["max_step"] <= 1
    assert v["mismatches"] <= max(1, 1e-4 * m * n)
    assert adopted <= max(1, 1e-4 * m * n)
    assert diff == 0
    # raw errors: float32 accumulation error, in grid steps
    Eimp = R.implied_errors_p(d["W"], R._values(codes, s, z), PA64, PB64)
    err_steps = np.abs(out["err"] - Eimp) / s[:, None]
    assert err_steps.max() < 1e-3, err_steps.max()
    dA, dB = np.diag(LA).astype(np.float64), np.diag(LB).astype(np.float64)
    obj_or = float(np.sum((dB[:, None] * E_or * dA[None, :]) ** 2))
    obj_self = float(np.sum((dB[:, None] * out["err"].astype(np.float64) * dA[None, :]) ** 2))
    assert out["objective"][0] == pytest.approx(obj_self, rel=1e-6)
    assert out["objective"][0] == pytest.approx(obj_or, rel=1e-3)


@pytest.mark.parametrize("m,n,seed", [(64, 64, 0), (128, 192, 1), (192, 128, 2), (320, 448, 3),
                                      (200, 136, 4), (130, 70, 5), (1, 64, 6), (64, 1, 7), (1, 1, 8),
                                      (7, 300, 9), (300, 7, 10), (65, 65, 11)])
def test_solve_isolated(m, n, seed):
    d = _problem(m, n, seed)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    LB, PB = fb["L"].astype(np.float32), fb["P"].astype(np.float32)
    out = gpu_solve(d, LA, PA, LB, PB)
    _check_solve(d, LA, PA, LB, PB, out, f"isolated seed={seed}")


def test_solve_isolated_1024():
    d = _problem(1024, 1024, 21)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    LB, PB = fb["L"].astype(np.float32), fb["P"].astype(np.float32)
    out = gpu_solve(d, LA, PA, LB, PB)
    _check_solve(d, LA, PA, LB, PB, out, "isolated 1024")


def test_solve_repeatable_and_stream_ordered():
    d = _problem(256, 320, 12)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    LB, PB = fb["L"].astype(np.float32), fb["P"].astype(np.float32)
    a = gpu_solve(d, LA, PA, LB, PB)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = gpu_solve(d, LA, PA, LB, PB)
    for k in ("codes", "V", "err", "objective"):
        assert np.array_equal(a[k], b[k]), k


def test_golden_grid_fixture_on_the_gpu():
    """The hand-worked fixture tests/golden/hand_grid_2x2.json (non-unit
    steps, fractional zero points, a clip at maxq, a clip at 0 and an exact
    half-way tie resolved to even; every value dyadic, so the float32 path is
    exact): the GPU's solve on the fixture's factors, its own factors and
    solve (no damping), and its one-sided path reproduce the hand-derived
    codes, values, errors and objectives exactly."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_grid_2x2.json")))
    f32 = lambda k: np.array(g[k], np.float32)   # noqa: E731
    d = {"W": f32("W"), "scale": f32("scale"), "zero": f32("zero"), "maxq": np.array(g["maxq"], np.int32)}
    out = gpu_solve(d, f32("L_A"), f32("P_A"), f32("L_B"), f32("P_B"))
    assert np.array_equal(out["codes"], np.array(g["codes"]))
    assert np.array_equal(out["V"], f32("V")) and np.array_equal(out["err"], f32("E"))
    assert out["objective"][0] == g["objective"]
    LA, PA, ia = gpu_factor(f32("A"), 0.0)
    LB, PB, ib = gpu_factor(f32("B"), 0.0)
    assert ia == 0 and ib == 0
    assert np.array_equal(LA, f32("L_A")) and np.array_equal(PA, f32("P_A"))
    assert np.array_equal(LB, f32("L_B")) and np.array_equal(PB, f32("P_B"))
    q = B.quantize(to_dev(d["W"]), to_dev(f32("A")), to_dev(f32("B")), to_dev(d["scale"]), to_dev(d["zero"]),
                   to_dev(d["maxq"]), 0.0, want_err=True)
    torch.cuda.synchronize()
    assert np.array_equal(q["codes"].cpu().numpy(), np.array(g["codes"]))
    assert np.array_equal(q["err"].cpu().numpy(), f32("E"))
    o = g["one_sided"]
    r = B.gptq(to_dev(d["W"]), to_dev(f32("L_A")), to_dev(f32("P_A")), to_dev(d["scale"]), to_dev(d["zero"]),
               to_dev(d["maxq"]), want_err=True)
    torch.cuda.synchronize()
    assert np.array_equal(r["codes"].cpu().numpy(), np.array(o["codes"]))
    assert np.array_equal(r["V"].cpu().numpy(), np.array(o["V"], np.float32))
    assert np.array_equal(r["err"].cpu().numpy(), np.array(o["E"], np.float32))
    assert r["objective"].item() == o["objective"]


# ---------------------------------------------------------- end to end

@pytest.mark.parametrize("m,n,seed", [(64, 64, 0), (256, 192, 1), (200, 330, 2)])
def test_end_to_end_small(m, n, seed):
    d = _problem(m, n, seed)
    LA, PA, ia = gpu_factor(d["A"])
    LB, PB, ib = gpu_factor(d["B"])
    assert ia == 0 and ib == 0
    out = gpu_solve(d, LA, PA, LB, PB)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    codes = out["codes"].astype(np.int64)
    v = R.validate(d["W"], codes, d["scale"], d["zero"], d["maxq"], fa["L"], fb["L"], tau=TAU)
    c_or, V_or, E_or = O2.bakron_recursive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    diff = int((codes != c_or).sum())
    print(f"end-to-end {m}x{n}: validator {v}, differing {diff}", flush=True)
    # GPU float32 factors vs the oracle's float64 ones: the bar is the count
    # (<= 1e-4 of the entries) and size (one step) of the mismatches.
    assert v["max_step"] <= 1 and v["mismatches"] <= max(1, 1e-4 * m * n)
    obj_g = R.objective(d["W"], out["V"], fa["L"], fb["L"])
    obj_o = R.objective(d["W"], V_or, fa["L"], fb["L"])
    assert obj_g == pytest.approx(obj_o, rel=1e-3)


# ------------------------------------------------------------ edge cases

def test_empty_inputs_are_noops():
    e = torch.empty((0, 5), dtype=torch.float32, device=DEV)
    out = B.solve(e, None, torch.eye(5, device=DEV), None, torch.empty((0, 0), device=DEV),
                  torch.empty(0, device=DEV), torch.empty(0, device=DEV),
                  torch.empty(0, dtype=torch.int32, device=DEV), want_objective=False)
    assert out["codes"].shape == (0, 5)
    L, P, info = B.factor(torch.empty((0, 0), dtype=torch.float32, device=DEV))
    assert L.shape == (0, 0)


def test_workspace_too_small_is_rejected():
    d = _problem(64, 64, 0)
    with pytest.raises(B.BakronError):
        B.solve(to_dev(d["W"]), None, torch.eye(64, device=DEV), None, torch.eye(64, device=DEV),
                to_dev(d["scale"]), to_dev(d["zero"]), to_dev(d["maxq"]), want_objective=False,
                ws=torch.empty(1024, dtype=torch.uint8, device=DEV))
