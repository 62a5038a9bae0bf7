"""Pins of the oracle's per-group grids (static groups of g input columns,
entry (i, j) rounded on grid [i][j // g] of an m x G array).

Pages: paper page "BaKron: Efficient Quantization with Kronecker-Factored
Hessians" (abstract: the base quantizer is modular); paper summary
"FastKron: Efficient Quantization with Kronecker-Factored Hessians"
(BaKron-naive, Theorem 3.2, Corollary 3.4).

What pins them, independently of the oracle's own indexing:
* a hand-worked fixture (tests/golden/hand_groups_2x4.json, derivation
  inside), which every form reproduces and which catches planted indexing
  mistakes (one grid per row, group j % g, transposed grid layout);
* Theorem 3.2 with grouped grids: brute-force GPTQ on vec(W) with the
  explicit Hessian equals every matrix-domain form;
* special cases: groups of g >= n, or groups whose grids are all equal, give
  the per-row result.
"""
import json
import os

import numpy as np
import pytest

from oracle import recursive as O2
from oracle import reference as R
from workloads import make_problem

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_groups_2x4.json")


def _fixture():
    g = json.load(open(GOLD))
    W = np.array(g["W"], np.float64)
    fa, fb = R.factor(np.array(g["A"]), g["damping"]), R.factor(np.array(g["B"]), g["damping"])
    grid = (np.array(g["scale"], np.float32), np.array(g["zero"], np.float32), np.array(g["maxq"], np.int32))
    return g, W, fa, fb, grid, g["group_size"]


def test_golden_groups_all_forms():
    g, W, fa, fb, (s, z, q), gs = _fixture()
    np.testing.assert_allclose(fa["P"], g["P_A"], atol=1e-15)
    m, n = W.shape
    runs = {
        "naive_col": R.bakron_naive(W, fa["P"], fb["P"], s, z, q, group_size=gs),
        "naive_row": R.bakron_naive(W, fa["P"], fb["P"], s, z, q, R.order_rowmajor(m, n), group_size=gs),
        "naive_anti": R.bakron_naive(W, fa["P"], fb["P"], s, z, q, R.order_antidiagonal(m, n), group_size=gs),
        "antidiagonal": R.bakron_antidiagonal(W, fa["P"], fb["P"], s, z, q, group_size=gs),
        "lform": R.bakron_lform(W, fa["L"], fb["L"], s, z, q, group_size=gs),
        "one_sided": R.gptq_columns(W, fa["P"], s, z, q, group_size=gs),
        "recursive_leaf1": O2.bakron_recursive(W, fa["P"], fb["P"], s, z, q, leaf=1, group_size=gs),
        "recursive_leaf3": O2.bakron_recursive(W, fa["P"], fb["P"], s, z, q, leaf=3, group_size=gs),
    }
    for name, (c, V, E) in runs.items():
        assert np.array_equal(c, g["codes"]), name
        np.testing.assert_allclose(V, g["V"], atol=1e-12, err_msg=name)
        np.testing.assert_allclose(E, g["E"], atol=1e-12, err_msg=name)
        assert R.objective_from_errors(E, fa["L"], fb["L"]) == pytest.approx(g["objective"], rel=1e-12)
    c, V = R.gptq_vectorized(W, fa["Ad"], fb["Ad"], s, z, q, group_size=gs)
    assert np.array_equal(c, g["codes"])
    assert R.objective(W, V, fa["L"], fb["L"]) == pytest.approx(g["objective"], rel=1e-12)
    v = R.validate(W, np.array(g["codes"]), s, z, q, fa["L"], fb["L"], group_size=gs)
    assert v["mismatches"] == 0


_ORIG = R.entry_grid


def _one_grid_per_row(s, z, maxq, m, n, group_size=None):
    return _ORIG(np.asarray(s)[:, 0], np.asarray(z)[:, 0], np.asarray(maxq)[:, 0], m, n, None)


def _group_mod(s, z, maxq, m, n, group_size=None):
    cols = np.arange(n) % group_size
    cols = np.minimum(cols, np.asarray(s).shape[1] - 1)
    return np.asarray(s)[:, cols], np.asarray(z)[:, cols], np.asarray(maxq)[:, cols]


def _transposed_layout(s, z, maxq, m, n, group_size=None):
    # reads the m x G grid as if it were stored G x m
    flat = lambda a: np.asarray(a).reshape(-1)   # noqa: E731
    G = np.asarray(s).shape[1]
    idx = (np.arange(n)[None, :] // group_size) * m + np.arange(m)[:, None]
    idx = np.minimum(idx, m * G - 1)
    return flat(s)[idx], flat(z)[idx], flat(maxq)[idx]


@pytest.mark.parametrize("plant", [_one_grid_per_row, _group_mod, _transposed_layout])
def test_golden_groups_catch_planted_indexing_mistakes(plant, monkeypatch):
    g, W, fa, fb, (s, z, q), gs = _fixture()
    monkeypatch.setattr(R, "entry_grid", plant)
    c, V, _ = R.bakron_naive(W, fa["P"], fb["P"], s, z, q, group_size=gs)
    same = np.array_equal(c, g["codes"]) and np.allclose(V, g["V"], rtol=0, atol=1e-12)
    assert not same, plant.__name__


# Theorem 3.2 with static per-group grids: the rounding rule of each entry is
# a fixed function of its working value, so every order gives GPTQ on vec(W).
@pytest.mark.parametrize("m,n,g,seed", [(7, 11, 3, 0), (16, 40, 8, 1), (5, 64, 16, 2), (1, 10, 4, 3),
                                        (33, 17, 5, 4), (40, 70, 32, 5)])
def test_groups_forms_agree(m, n, g, seed):
    d = make_problem(m, n, seed, group_size=g)
    assert d["scale"].shape == (m, -(-n // g))
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    W, s, z, q = d["W"], d["scale"], d["zero"], d["maxq"]
    c0, V0, E0 = R.bakron_naive(W, fa["P"], fb["P"], s, z, q, group_size=g)
    forms = [R.bakron_naive(W, fa["P"], fb["P"], s, z, q, R.order_rowmajor(m, n), group_size=g),
             R.bakron_naive(W, fa["P"], fb["P"], s, z, q, R.order_antidiagonal(m, n), group_size=g),
             R.bakron_antidiagonal(W, fa["P"], fb["P"], s, z, q, group_size=g),
             R.bakron_lform(W, fa["L"], fb["L"], s, z, q, group_size=g)]
    forms += [O2.bakron_recursive(W, fa["P"], fb["P"], s, z, q, leaf=lf, group_size=g) for lf in (1, 5, 32)]
    for c, V, E in forms:
        assert np.array_equal(c, c0)
        np.testing.assert_allclose(V, V0, rtol=0, atol=1e-12)
    if m * n <= 4096:
        c, V = R.gptq_vectorized(W, fa["Ad"], fb["Ad"], s, z, q, group_size=g)
        assert np.array_equal(c, c0)
    v = R.validate(W, c0, s, z, q, PA=fa["P"], PB=fb["P"], group_size=g)
    assert v["mismatches"] == 0


def test_groups_reduce_to_per_row():
    # a group wider than the row, and groups whose grids all equal the row's
    d = make_problem(24, 50, 7)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    W, s, z, q = d["W"], d["scale"], d["zero"], d["maxq"]
    c_row = R.bakron_naive(W, fa["P"], fb["P"], s, z, q)[0]
    c_wide = R.bakron_naive(W, fa["P"], fb["P"], s[:, None], z[:, None], q[:, None], group_size=64)[0]
    assert np.array_equal(c_wide, c_row)
    G = -(-50 // 8)
    rep = lambda a: np.repeat(a[:, None], G, axis=1)   # noqa: E731
    c_rep = O2.bakron_recursive(W, fa["P"], fb["P"], rep(s), rep(z), rep(q), group_size=8)[0]
    assert np.array_equal(c_rep, c_row)


def test_groups_one_sided_and_follow():
    d = make_problem(30, 70, 9, group_size=16)
    fa = R.factor(d["A"])
    W, s, z, q = d["W"], d["scale"], d["zero"], d["maxq"]
    c1, V1, E1 = R.gptq_columns(W, fa["P"], s, z, q, group_size=16)
    c2, V2, E2 = R.bakron_naive(W, fa["P"], np.eye(30), s, z, q, group_size=16)
    assert np.array_equal(c1, c2)
    np.testing.assert_allclose(E1, E2, atol=1e-12)
    rows = np.array([3, 29, 11])
    cs, _, Es = R.gptq_columns(W, fa["P"], s, z, q, rows=rows, group_size=16)
    assert np.array_equal(cs, c1[rows]) and np.array_equal(Es, E1[rows])
    c3, _, _, k = R.gptq_columns(W, fa["P"], s, z, q, follow=c1, tau=0.5, group_size=16)
    assert k == 0 and np.array_equal(c3, c1)
    v = R.validate(W, c1, s, z, q, PA=fa["P"], PB=None, group_size=16)
    assert v["mismatches"] == 0
    flip = c1.copy()
    flip[5, 40] = flip[5, 40] + 1 if flip[5, 40] < q[5, 2] else flip[5, 40] - 1
    assert R.validate(W, flip, s, z, q, PA=fa["P"], PB=None, group_size=16)["bad"] >= 1


def test_group_grid_recipe():
    # each group's grid spans its own slice of the original row exactly
    d = make_problem(6, 20, 2, bits=2, group_size=8)
    W, s, z, q = d["W"].astype(np.float64), d["scale"], d["zero"], d["maxq"]
    assert s.shape == (6, 3) and np.all(q == 3)
    for k in range(3):
        sl = W[:, 8 * k:8 * (k + 1)]
        np.testing.assert_allclose(s[:, k], (sl.max(1) - sl.min(1)) / 3, rtol=1e-6)
        np.testing.assert_allclose(z[:, k] * s[:, k], -sl.min(1), rtol=1e-5, atol=1e-9)
