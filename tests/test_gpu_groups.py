"""GPU parity of the per-group grids (bakron_solve_grouped, bakron_gptq_grouped,
through the C ABI) against the float64 oracle's grouped forms.

Pages: paper page "BaKron: Efficient Quantization with Kronecker-Factored
Hessians" (abstract: the base quantizer is modular); paper summary
"FastKron: Efficient Quantization with Kronecker-Factored Hessians"
(Theorem 3.2, Corollary 3.4).

Static groups of g input columns (g a multiple of 64 on the GPU), grids from
the original W's group slices.  The bar is the per-row one: the oracle on the
same factors, following the GPU's code only where its own decision lies
within TAU grid steps of a rounding boundary, gives every code equal (at most
1e-4 of the entries followed); the validator finds no mismatch outside that
band; V is s (c - z) bit for bit; raw errors within 1e-3 grid steps; the
objective within 1e-3.
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


def _expected_values(d, codes, g):
    m, n = codes.shape
    S, Z, _ = R.entry_grid(d["scale"], d["zero"], d["maxq"], m, n, g)
    return (S * (codes.astype(np.float32) - Z)).astype(np.float32), S


def _check(d, g, PA, PB, out, label, follow_rows=None):
    m, n = d["W"].shape
    s, z, q = d["scale"], d["zero"], d["maxq"]
    codes = out["codes"].astype(np.int64)
    Vexp, S = _expected_values(d, codes, g)
    assert np.array_equal(out["V"], Vexp), label
    v = R.validate(d["W"], codes, s, z, q, tau=TAU, PA=PA.astype(np.float64),
                   PB=None if PB is None else PB.astype(np.float64), return_errors=True, group_size=g)
    E = v.pop("E")
    v.pop("tie_mask"), v.pop("bad_mask")
    print(f"{label}: {m}x{n} g={g} validator {v}", flush=True)
    assert v["bad"] == 0 and v["max_step"] <= 1
    assert v["mismatches"] <= max(1, 1e-4 * m * n)
    assert (np.abs(out["err"] - E) / S).max() < 1e-3
    if PB is None:
        rows = np.arange(m) if follow_rows is None else follow_rows
        c_or, _, E_or, adopted = R.gptq_columns(d["W"], PA.astype(np.float64), s, z, q, rows=rows,
                                                follow=codes[rows], tau=TAU, group_size=g)
        diff = int((codes[rows] != c_or).sum())
    else:
        c_or, _, E_or, adopted = O2.bakron_recursive(d["W"], PA.astype(np.float64), PB.astype(np.float64), s, z, q,
                                                     follow=codes, tau=TAU, group_size=g)
        diff = int((codes != c_or).sum())
    print(f"{label}: oracle adopted {adopted}, {diff} codes differ", flush=True)
    assert adopted <= max(1, 1e-4 * m * n) and diff == 0
    return E_or


SHAPES = [(128, 192, 64, 0), (130, 200, 64, 1), (96, 300, 128, 2), (1, 256, 64, 3), (200, 136, 128, 4),
          (64, 64, 64, 5), (320, 448, 192, 6)]


@pytest.mark.parametrize("m,n,g,seed", SHAPES)
def test_solve_grouped_matches_oracle(m, n, g, seed):
    d = make_problem(m, n, 200 + seed, group_size=g)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    LB, PB = fb["L"].astype(np.float32), fb["P"].astype(np.float32)
    out = B.solve(to_dev(d["W"]), to_dev(LA), to_dev(PA), to_dev(LB), to_dev(PB), to_dev(d["scale"]),
                  to_dev(d["zero"]), to_dev(d["maxq"]), want_err=True, group_size=g)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    E_or = _check(d, g, PA, PB, out, "solve_grouped")
    dA, dB = np.diag(LA).astype(np.float64), np.diag(LB).astype(np.float64)
    assert out["objective"][0] == pytest.approx(float(np.sum((dB[:, None] * E_or * dA[None, :]) ** 2)), rel=1e-3)


@pytest.mark.parametrize("m,n,g,seed", SHAPES)
def test_gptq_grouped_matches_oracle(m, n, g, seed):
    d = make_problem(m, n, 300 + seed, group_size=g)
    fa = R.factor(d["A"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    out = B.gptq(to_dev(d["W"]), to_dev(LA), to_dev(PA), to_dev(d["scale"]), to_dev(d["zero"]), to_dev(d["maxq"]),
                 want_err=True, group_size=g)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in out.items()}
    E_or = _check(d, g, PA, None, out, "gptq_grouped")
    dA = np.diag(LA).astype(np.float64)
    assert out["objective"][0] == pytest.approx(float(np.sum((E_or * dA[None, :]) ** 2)), rel=1e-3)


def test_one_group_equals_per_row():
    # a group at least as wide as the row: the per-row calls, bit for bit
    d = make_problem(192, 200, 7)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    T = {k: to_dev(v) for k, v in (("W", d["W"]), ("LA", fa["L"].astype(np.float32)), ("PA", fa["P"].astype(np.float32)),
                                   ("LB", fb["L"].astype(np.float32)), ("PB", fb["P"].astype(np.float32)))}
    s, z, q = to_dev(d["scale"]), to_dev(d["zero"]), to_dev(d["maxq"])
    a = B.solve(T["W"], T["LA"], T["PA"], T["LB"], T["PB"], s, z, q, want_err=True)
    b = B.solve(T["W"], T["LA"], T["PA"], T["LB"], T["PB"], s[:, None].contiguous(), z[:, None].contiguous(),
                q[:, None].contiguous(), want_err=True, group_size=256)
    c = B.gptq(T["W"], T["LA"], T["PA"], s, z, q, want_err=True)
    e = B.gptq(T["W"], T["LA"], T["PA"], s[:, None].contiguous(), z[:, None].contiguous(), q[:, None].contiguous(),
               want_err=True, group_size=1024)
    torch.cuda.synchronize()
    for key in ("codes", "V", "err", "objective"):
        assert torch.equal(a[key], b[key]) and torch.equal(c[key], e[key]), key


def test_grouped_full_size():
    """The 4096 x 4096 Student-t layer with groups of 128 columns (2 bits):
    the two-sided solve on the GPU's own factors against the oracle on the
    same factors at every entry, and the one-sided call on every row through
    the validator (sampled rows through the oracle)."""
    spec = WL.by_name("sq4096_t5")
    d = WL.generate(spec, group_size=128)
    print(f"grouped full size: {spec.m}x{spec.n} g=128", flush=True)
    LA, PA, ia = B.factor(to_dev(d["A"]), 0.01)
    LB, PB, ib = B.factor(to_dev(d["B"]), 0.01)
    W, s, z, q = to_dev(d["W"]), to_dev(d["scale"]), to_dev(d["zero"]), to_dev(d["maxq"])
    out = B.solve(W, LA, PA, LB, PB, s, z, q, want_err=True, group_size=128)
    one = B.gptq(W, LA, PA, s, z, q, want_err=True, group_size=128)
    torch.cuda.synchronize()
    assert int(ia.item()) == 0 and int(ib.item()) == 0
    PA, PB = PA.cpu().numpy(), PB.cpu().numpy()
    _check(d, 128, PA, PB, {k: v.cpu().numpy() for k, v in out.items()}, "solve_grouped 4096")
    rows = np.unique(np.concatenate([[0, spec.m - 1], np.random.default_rng(4).choice(spec.m, 30, replace=False)]))
    _check(d, 128, PA, None, {k: v.cpu().numpy() for k, v in one.items()}, "gptq_grouped 4096", follow_rows=rows)
