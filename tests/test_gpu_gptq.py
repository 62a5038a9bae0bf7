"""GPU parity of the one-sided case B = I (bakron_gptq, through the C ABI)
against the float64 oracle.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (setup: GPTQ's Hessian is A (x) I; derivation:
BaKron-naive); [N5] (GPTQ as the one-sided comparison point).

With B = I rows are independent, so the oracle (``gptq_columns``) can be run
on any subset of rows: full-size workloads are checked on sampled rows.
Tolerances are those of the two-sided solve: codes equal the rounding of the
value they were rounded from except within TAU grid steps of a boundary (at
most 1e-4 of the entries, one step); the oracle on the same factors, taking
over the GPU's code wherever its own decision lies within TAU of a boundary,
gives every code equal; raw errors within 1e-3 grid steps; objective within
1e-3 relative.
"""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B
import workloads as WL
from oracle import reference as R
from workloads import make_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TAU = 1e-4


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_gptq(d, LA, PA, **kw):
    out = B.gptq(to_dev(d["W"]), to_dev(LA), to_dev(PA), to_dev(d["scale"]), to_dev(d["zero"]),
                 to_dev(d["maxq"]), want_err=True, **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_rows(d, PA32, out, rows, label):
    """Validator, same-factor oracle and error checks on the given rows."""
    s, z, mq = d["scale"][rows], d["zero"][rows], d["maxq"][rows]
    W = d["W"][rows]
    codes = out["codes"][rows].astype(np.int64)
    n = W.shape[1]
    assert np.all(codes <= mq[:, None]), label
    Vexp = (s[:, None] * (codes.astype(np.float32) - z[:, None])).astype(np.float32)
    assert np.array_equal(out["V"][rows], Vexp), label
    PA64 = PA32.astype(np.float64)
    v = R.validate(W, codes, s, z, mq, tau=TAU, PA=PA64, PB=np.eye(len(rows)), return_errors=True)
    E, ties = v.pop("E"), v.pop("tie_mask")
    v.pop("bad_mask")
    print(f"{label}: validator {v}", flush=True)
    assert v["bad"] == 0 and v["max_step"] <= 1
    assert v["mismatches"] <= max(1, 1e-4 * W.size)
    steps = np.abs(out["err"][rows] - E) / s[:, None]
    assert steps.max() < 1e-3, steps.max()
    # the oracle on the same factors, following the GPU at near-ties (within
    # TAU of a rounding boundary both roundings are valid): every code equal
    c_or, V_or, E_or, adopted = R.gptq_columns(d["W"], PA64, d["scale"], d["zero"], d["maxq"], rows=rows,
                                               follow=codes, tau=TAU)
    diff = int((codes != c_or).sum())
    print(f"{label}: oracle adopted {adopted} near-tie codes; {diff} codes differ", flush=True)
    assert adopted <= max(1, 1e-4 * W.size)
    assert diff == 0
    return E_or, adopted


SHAPES = [(64, 64, 0), (96, 200, 1), (130, 70, 2), (1, 64, 3), (64, 1, 4), (7, 300, 5), (300, 7, 6),
          (65, 65, 7), (32, 1000, 8), (2, 2, 9), (256, 640, 10)]


@pytest.mark.parametrize("m,n,seed", SHAPES)
def test_gptq_matches_oracle(m, n, seed):
    d = make_problem(m, n, seed, global_grid=(n <= 2))
    fa = R.factor(d["A"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    out = gpu_gptq(d, LA, PA)
    rows = np.arange(m)
    E_or, adopted = check_rows(d, PA, out, rows, f"gptq {m}x{n}")
    dA = np.diag(LA).astype(np.float64)
    obj_self = float(np.sum((out["err"].astype(np.float64) * dA[None, :]) ** 2))
    assert out["objective"][0] == pytest.approx(obj_self, rel=1e-6)
    obj_or = float(np.sum((E_or * np.diag(fa["L"])[None, :]) ** 2))
    assert out["objective"][0] == pytest.approx(obj_or, rel=1e-3)


def test_gptq_equals_two_sided_solve_with_identity_b():
    # bakron_solve with P_B = L_B = I is the same rounding (B = I); the two
    # paths sum in different orders, so codes may part only at ties
    m, n = 192, 320
    d = make_problem(m, n, 31)
    fa = R.factor(d["A"])
    LA, PA = fa["L"].astype(np.float32), fa["P"].astype(np.float32)
    I = np.eye(m, dtype=np.float32)
    g = gpu_gptq(d, LA, PA)
    out = B.solve(to_dev(d["W"]), to_dev(LA), to_dev(PA), to_dev(I), to_dev(I), to_dev(d["scale"]),
                  to_dev(d["zero"]), to_dev(d["maxq"]))
    torch.cuda.synchronize()
    c2 = out["codes"].cpu().numpy()
    ties = np.zeros((m, n), bool)
    for c in (g["codes"], c2):
        v = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], tau=TAU, PA=PA.astype(np.float64),
                       PB=np.eye(m), return_errors=True)
        assert v["bad"] == 0
        ties |= v["tie_mask"]
    outside = ~R.dependency_cone(ties)
    assert np.array_equal(g["codes"][outside], c2[outside])
    assert float(out["objective"].item()) == pytest.approx(float(g["objective"][0]), rel=1e-3)


@pytest.mark.parametrize("name", ["sq4096_t5", "sq8192_mixed"])
def test_gptq_full_size(name):
    """Every row through the validator (rows are independent, P_B = I), and
    sampled rows through the oracle in tie-following mode."""
    spec = WL.by_name(name)
    d = WL.generate(spec)
    m, n = spec.m, spec.n
    print(f"gptq config {name}: {m}x{n}", flush=True)
    LA, PA, info = B.factor(to_dev(d["A"]), 0.01)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    LA, PA = LA.cpu().numpy(), PA.cpu().numpy()
    out = gpu_gptq(d, LA, PA)
    s, z, mq = d["scale"], d["zero"], d["maxq"]
    codes = out["codes"].astype(np.int64)
    assert np.all(codes <= mq[:, None])
    assert np.array_equal(out["V"], (s[:, None] * (codes.astype(np.float32) - z[:, None])).astype(np.float32))
    v = R.validate(d["W"], codes, s, z, mq, tau=TAU, PA=PA.astype(np.float64), PB=None, return_errors=True)
    E = v.pop("E")
    v.pop("tie_mask"), v.pop("bad_mask")
    print(f"gptq {name}: validator over all {m} rows {v}", flush=True)
    assert v["bad"] == 0 and v["max_step"] <= 1
    assert v["mismatches"] <= max(1, 1e-4 * m * n)
    assert (np.abs(out["err"] - E) / s[:, None]).max() < 1e-3
    del E
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, m - 1], rng.choice(m, size=30, replace=False)]))
    check_rows(d, PA, out, rows, f"gptq {name} rows {len(rows)}")
    dA = np.diag(LA).astype(np.float64)
    obj_self = float(np.sum((out["err"].astype(np.float64) * dA[None, :]) ** 2))
    assert out["objective"][0] == pytest.approx(obj_self, rel=1e-6)


def test_gptq_empty_and_bad_workspace():
    d = make_problem(64, 64, 2)
    fa = R.factor(d["A"])
    LA, PA = to_dev(fa["L"].astype(np.float32)), to_dev(fa["P"].astype(np.float32))
    lib = B.lib()
    assert lib.bakron_gptq(None, 0, 64, None, None, None, None, None, None, None, None, None, None, 0,
                           None) == 0
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.BakronError) as ei:
        B.gptq(to_dev(d["W"]), LA, PA, to_dev(d["scale"]), to_dev(d["zero"]), to_dev(d["maxq"]), ws=ws)
    assert ei.value.code == -3
