"""Pins of the float64 oracle against facts fixed by the pages and by
mathematics -- not against the oracle itself.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (setup, derivation, Theorem 3.2, Corollary 3.4);
[N5] news article "BaKron Reduces Two-Sided Hessian Quantization to Cubic
Complexity, With Its 8192-Square-Matrix Kernel 60x Faster Than YAQA"
(GPTQ = A (x) I).
"""
import json
import os

import numpy as np
import pytest

from oracle import reference as R
from oracle import recursive as O2
from workloads import make_problem

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _factors(d, frac=0.01):
    return R.factor(d["A"], frac), R.factor(d["B"], frac)


def _all_forms(d, fa, fb):
    W, s, z, mq = d["W"], d["scale"], d["zero"], d["maxq"]
    m, n = W.shape
    out = {}
    if m * n <= 4096:
        out["vec_bruteforce"] = R.gptq_vectorized(W, fa["Ad"], fb["Ad"], s, z, mq)[:2]
    out["naive_col"] = R.bakron_naive(W, fa["P"], fb["P"], s, z, mq, R.order_colmajor(m, n))[:2]
    out["naive_row"] = R.bakron_naive(W, fa["P"], fb["P"], s, z, mq, R.order_rowmajor(m, n))[:2]
    out["naive_anti"] = R.bakron_naive(W, fa["P"], fb["P"], s, z, mq, R.order_antidiagonal(m, n))[:2]
    out["antidiagonal"] = R.bakron_antidiagonal(W, fa["P"], fb["P"], s, z, mq)[:2]
    out["lform"] = R.bakron_lform(W, fa["L"], fb["L"], s, z, mq)[:2]
    for leaf in (1, 5, 32):
        c, V, _ = O2.bakron_recursive(W, fa["P"], fb["P"], s, z, mq, leaf=leaf)
        out[f"recursive_leaf{leaf}"] = (c.astype(np.float64), V)
    return out


# Theorem 3.2 ([S]): naive, antidiagonal, recursive and BaKron give the same
# output; all equal GPTQ on vec(W) with the explicit Hessian (BaKron-naive's
# definition).  Shapes cover non-square, m = 1, n = 1 and non-multiples of
# the recursive leaf size.
@pytest.mark.parametrize("m,n,seed", [(7, 5, 0), (16, 16, 1), (40, 70, 2), (64, 64, 3),
                                      (1, 9, 4), (33, 17, 6), (5, 64, 8)])
def test_forms_agree(m, n, seed):
    d = make_problem(m, n, seed)
    fa, fb = _factors(d)
    forms = _all_forms(d, fa, fb)
    c0, V0 = forms["naive_col"]
    for name, (c, V) in forms.items():
        assert np.array_equal(c, c0), name
        np.testing.assert_allclose(V, V0, rtol=0, atol=1e-12, err_msg=name)


def test_forms_agree_n1():
    d = make_problem(9, 1, 5, global_grid=True)
    fa, fb = _factors(d)
    forms = _all_forms(d, fa, fb)
    c0, _ = forms["vec_bruteforce"]
    for name, (c, _) in forms.items():
        assert np.array_equal(c, c0), name


def test_recursive_matches_naive_1024():
    d = make_problem(256, 320, 11)
    fa, fb = _factors(d)
    c1, V1, E1 = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    c2, V2, E2 = O2.bakron_recursive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    assert np.array_equal(c1, c2)
    np.testing.assert_allclose(E2, E1, rtol=0, atol=1e-12)


# Hand-worked fixtures (tests/golden/*.json, derivations inside).
@pytest.mark.parametrize("name", ["hand_1x2.json", "hand_2x2.json", "hand_grid_2x2.json"])
def test_golden_hand_examples(name):
    g = json.load(open(os.path.join(GOLD, name)))
    W = np.array(g["W"], dtype=np.float64)
    A = np.array(g["A"], dtype=np.float64)
    B = np.array(g["B"], dtype=np.float64)
    s = np.array(g["scale"], np.float32)
    z = np.array(g["zero"], np.float32)
    mq = np.array(g["maxq"], np.int32)
    fa, fb = R.factor(A, g["damping"]), R.factor(B, g["damping"])
    if "L_A" in g:
        np.testing.assert_allclose(fa["L"], g["L_A"], atol=1e-15)
        np.testing.assert_allclose(fa["P"], g["P_A"], atol=1e-15)
    if "L_B" in g:
        np.testing.assert_allclose(fb["L"], g["L_B"], atol=1e-15)
        np.testing.assert_allclose(fb["P"], g["P_B"], atol=1e-15)
    for c, V, E in [R.bakron_naive(W, fa["P"], fb["P"], s, z, mq),
                    R.bakron_naive(W, fa["P"], fb["P"], s, z, mq, R.order_rowmajor(*W.shape)),
                    R.bakron_antidiagonal(W, fa["P"], fb["P"], s, z, mq),
                    R.bakron_lform(W, fa["L"], fb["L"], s, z, mq),
                    O2.bakron_recursive(W, fa["P"], fb["P"], s, z, mq, leaf=1)]:
        assert np.array_equal(c, g["codes"])
        np.testing.assert_allclose(V, g["V"], atol=1e-12)
        np.testing.assert_allclose(E, g["E"], atol=1e-12)
        assert R.objective(W, V, fa["L"], fb["L"]) == pytest.approx(g["objective"], rel=1e-12)
        assert R.objective_from_errors(E, fa["L"], fb["L"]) == pytest.approx(g["objective"], rel=1e-12)
    c, V = R.gptq_vectorized(W, fa["Ad"], fb["Ad"], s, z, mq)
    assert np.array_equal(c, g["codes"])
    np.testing.assert_allclose(V, g["V"], atol=1e-12)
    # tie following on its own codes adopts nothing, even at the exact tie
    c2, _, _, k = O2.bakron_recursive(W, fa["P"], fb["P"], s, z, mq, leaf=1, follow=np.array(g["codes"]))
    assert k == 0 and np.array_equal(c2, g["codes"])
    v = R.validate(W, np.array(g["codes"]), s, z, mq, fa["L"], fb["L"])
    assert v["mismatches"] == 0


def _grid_fixture():
    g = json.load(open(os.path.join(GOLD, "hand_grid_2x2.json")))
    W = np.array(g["W"], dtype=np.float64)
    fa, fb = R.factor(np.array(g["A"]), g["damping"]), R.factor(np.array(g["B"]), g["damping"])
    return g, W, fa, fb, np.array(g["scale"], np.float32), np.array(g["zero"], np.float32), \
        np.array(g["maxq"], np.int32)


def test_golden_grid_example_one_sided():
    """The fixture's B = I case (hand-worked in the fixture): the one-sided
    form, BaKron-naive with P_B = I and textbook GPTQ all reproduce it."""
    g, W, fa, _, s, z, mq = _grid_fixture()
    o = g["one_sided"]
    c, V, E = R.gptq_columns(W, fa["P"], s, z, mq)
    assert np.array_equal(c, o["codes"])
    np.testing.assert_allclose(V, o["V"], atol=1e-12)
    np.testing.assert_allclose(E, o["E"], atol=1e-12)
    assert R.objective_from_errors(E, fa["L"], np.eye(2)) == pytest.approx(o["objective"], rel=1e-12)
    c2, _, E2 = R.bakron_naive(W, fa["P"], np.eye(2), s, z, mq)
    assert np.array_equal(c2, o["codes"]) and np.allclose(E2, o["E"], atol=1e-12)
    assert np.array_equal(_textbook_gptq_rows(W, fa["Ad"], s, z, mq), o["codes"])


def _quant_half_up(w, s, z, maxq):
    x = (np.asarray(w, np.float64).astype(np.float32) / np.asarray(s, np.float32)).astype(np.float32) \
        + np.asarray(z, np.float32)
    c = np.clip(np.floor(x.astype(np.float64) + 0.5), 0, np.asarray(maxq, np.float64))
    return c, np.asarray(s, np.float64) * (c - np.asarray(z, np.float64))


def _quant_no_upper_clip(w, s, z, maxq):
    return _ORIG_QUANT(w, s, z, np.full(np.shape(maxq), 10 ** 6))


def _quant_no_lower_clip(w, s, z, maxq):
    x = (np.asarray(w, np.float64).astype(np.float32) / np.asarray(s, np.float32)).astype(np.float32) \
        + np.asarray(z, np.float32)
    c = np.minimum(np.rint(x), np.asarray(maxq)).astype(np.float64)
    return c, np.asarray(s, np.float64) * (c - np.asarray(z, np.float64))


def _quant_integer_zero(w, s, z, maxq):
    return _ORIG_QUANT(w, s, np.rint(np.asarray(z, np.float32)), maxq)


def _quant_unit_step(w, s, z, maxq):
    return _ORIG_QUANT(w, np.ones_like(np.asarray(s, np.float32)), z, maxq)


_ORIG_QUANT = R.quantize


# Mistakes planted in the oracle's base quantizer (on the CPU): each one of
# them changes the hand-worked fixture's codes, so the fixture pins every
# branch of the rounding rule.
@pytest.mark.parametrize("plant", [_quant_half_up, _quant_no_upper_clip, _quant_no_lower_clip,
                                   _quant_integer_zero, _quant_unit_step])
def test_golden_grid_example_catches_planted_quantizer_mistakes(plant, monkeypatch):
    g, W, fa, fb, s, z, mq = _grid_fixture()
    monkeypatch.setattr(R, "quantize", plant)
    c, V, _ = R.bakron_naive(W, fa["P"], fb["P"], s, z, mq)
    same = np.array_equal(c, g["codes"]) and np.allclose(V, g["V"], rtol=0, atol=1e-12)
    assert not same, plant.__name__


# RevCholesky ([S] Corollary 3.4): A_d = L^T L, L lower with positive diagonal.
@pytest.mark.parametrize("n,seed", [(1, 0), (5, 1), (64, 2), (130, 3)])
def test_rev_cholesky_definition(n, seed):
    d = make_problem(4, n, seed, global_grid=True)
    f = R.factor(d["A"])
    L = f["L"]
    assert np.array_equal(L, np.tril(L))
    assert np.all(np.diag(L) > 0)
    np.testing.assert_allclose(L.T @ L, f["Ad"], rtol=0, atol=1e-12 * np.abs(f["Ad"]).max())
    # bottom-up elimination written from A = L^T L, row n-1 first
    A = f["Ad"].copy()
    L2 = np.zeros_like(A)
    for k in range(n - 1, -1, -1):
        L2[k, k] = np.sqrt(A[k, k])
        L2[k, :k] = A[k, :k] / L2[k, k]
        A[:k, :k] -= np.outer(L2[k, :k], L2[k, :k])
    np.testing.assert_allclose(L, L2, rtol=1e-10, atol=1e-12)
    P = f["P"]
    assert np.allclose(np.diag(P), 1.0) and np.array_equal(P, np.tril(P))
    np.testing.assert_allclose(L @ (P / np.diag(L)[None, :]), np.eye(n), atol=1e-9)


@pytest.mark.parametrize("n,seed", [(5, 1), (64, 2), (130, 3)])
def test_factor_float32_is_a_float32_factorisation(n, seed):
    # float32 arrays out, A_d = L^T L within float32 backward error, the
    # float64 factor within float32 forward error, unit diagonal of P
    d = make_problem(4, n, seed, global_grid=True)
    f32, f64 = R.factor_float32(d["A"]), R.factor(d["A"])
    assert f32["L"].dtype == np.float32 and f32["P"].dtype == np.float32
    L = f32["L"].astype(np.float64)
    assert np.array_equal(L, np.tril(L)) and np.all(np.diag(L) > 0)
    u = 2.0 ** -24
    Ad = f64["Ad"]
    assert np.linalg.norm(L.T @ L - Ad) <= 10 * n * u * np.linalg.norm(Ad)
    np.testing.assert_allclose(np.diag(f32["P"]), 1.0, atol=4 * u)
    kappa = np.linalg.cond(Ad)
    assert np.linalg.norm(f32["P"] - f64["P"]) <= 10 * n * u * kappa * np.linalg.norm(f64["P"])


def test_rev_cholesky_rejects_indefinite():
    A = np.array([[1.0, 2.0], [2.0, 1.0]])
    with pytest.raises(np.linalg.LinAlgError):
        R.rev_cholesky(A)


def test_damping_reading():
    A = np.diag([1.0, 3.0])
    np.testing.assert_allclose(R.damp(A, 0.01), np.diag([1.02, 3.02]))


# Objective identity: ||L(B)(V-W)L(A)^T||^2 = sum (L_B,ii L_A,jj e_ij)^2.
@pytest.mark.parametrize("m,n,seed", [(12, 9, 0), (64, 40, 1)])
def test_objective_identity(m, n, seed):
    d = make_problem(m, n, seed)
    fa, fb = _factors(d)
    c, V, E = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    a = R.objective(d["W"], V, fa["L"], fb["L"])
    b = R.objective_from_errors(E, fa["L"], fb["L"])
    assert a == pytest.approx(b, rel=1e-12)
    np.testing.assert_allclose(R.implied_errors(d["W"], V, fa["L"], fb["L"]), E, atol=1e-12)


# Corollary 3.4 ([S]): with unit grid step and no clipping,
# ||L(B)(V-W)L(A)^T||_F^2 <= tr(A) tr(B) / 4; per-row steps generalise it to
# sum_i s_i^2 L_B,ii^2 / 4 * sum_j L_A,jj^2.
@pytest.mark.parametrize("seed", range(6))
def test_corollary_3_4_bound(seed):
    rng = np.random.default_rng(100 + seed)
    m, n = 11, 13
    d = make_problem(m, n, seed)
    fa, fb = _factors(d)
    W = rng.standard_normal((m, n)) * 3.0
    s = np.ones(m, np.float32)
    z = np.full(m, 1000.0, np.float32)          # codes far from 0 and maxq: no clipping
    mq = np.full(m, 2000, np.int32)
    c, V, E = R.bakron_naive(W, fa["P"], fb["P"], s, z, mq)
    assert np.all((c > 0) & (c < 2000))
    obj = R.objective(W, V, fa["L"], fb["L"])
    assert obj <= 0.25 * np.trace(fa["Ad"]) * np.trace(fb["Ad"])
    assert obj <= 0.25 * np.sum(np.diag(fb["L"]) ** 2) * np.sum(np.diag(fa["L"]) ** 2) * (1 + 1e-12)
    s2 = np.exp(rng.standard_normal(m)).astype(np.float32)
    c, V, E = R.bakron_naive(W, fa["P"], fb["P"], s2, z, mq)
    bound = 0.25 * np.sum(s2.astype(float) ** 2 * np.diag(fb["L"]) ** 2) * np.sum(np.diag(fa["L"]) ** 2)
    assert R.objective(W, V, fa["L"], fb["L"]) <= bound * (1 + 1e-12)


def _textbook_gptq_rows(W, H, s, z, mq):
    """GPTQ (one-sided) as usually stated: columns in order, H^-1 = U^T U,
    quantize column j, err = (w - q)/U_jj, later columns -= err * U_j,later."""
    W = np.array(W, dtype=np.float64)
    m, n = W.shape
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    Q = np.zeros_like(W)
    for j in range(n):
        x = (W[:, j].astype(np.float32) / s).astype(np.float32) + z
        q = np.clip(np.rint(x), 0, mq).astype(np.float64)
        Q[:, j] = q
        err = (W[:, j] - s.astype(np.float64) * (q - z.astype(np.float64))) / U[j, j]
        W[:, j:] -= np.outer(err, U[j, j:])
    return Q


# GPTQ special case ([S] setup; [N5]): B = I gives row-wise textbook GPTQ
# with Hessian A; A = I gives column-wise GPTQ with Hessian B.
def test_special_case_B_identity_is_gptq():
    d = make_problem(20, 48, 3)
    fa = R.factor(d["A"])
    fb = R.factor(np.eye(20))
    c, _, _ = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    g = _textbook_gptq_rows(d["W"], fa["Ad"], d["scale"], d["zero"], d["maxq"])
    assert np.array_equal(c, g)


def test_gptq_columns_is_textbook_gptq():
    # the column-by-column form of the case B = I against textbook GPTQ
    # (Cholesky of the inverse Hessian), an independent formula path
    d = make_problem(24, 80, 13)
    fa = R.factor(d["A"])
    c, V, E = R.gptq_columns(d["W"], fa["P"], d["scale"], d["zero"], d["maxq"])
    g = _textbook_gptq_rows(d["W"], fa["Ad"], d["scale"], d["zero"], d["maxq"])
    assert np.array_equal(c, g)
    np.testing.assert_allclose(V, R._values(c, d["scale"], d["zero"]), rtol=0, atol=1e-15)


def test_gptq_columns_is_bakron_with_identity_b():
    # same codes, values and errors as BaKron-naive with P_B = I, in the
    # anti-diagonal order (Theorem 3.2: any linear extension)
    d = make_problem(18, 40, 14)
    fa = R.factor(d["A"])
    PB = np.eye(18)
    c1, V1, E1 = R.gptq_columns(d["W"], fa["P"], d["scale"], d["zero"], d["maxq"])
    c2, V2, E2 = R.bakron_naive(d["W"], fa["P"], PB, d["scale"], d["zero"], d["maxq"],
                                order=R.order_antidiagonal(18, 40))
    assert np.array_equal(c1, c2)
    np.testing.assert_allclose(E1, E2, rtol=0, atol=1e-12)


def test_gptq_columns_rows_are_independent():
    d = make_problem(30, 50, 15)
    fa = R.factor(d["A"])
    c, V, E = R.gptq_columns(d["W"], fa["P"], d["scale"], d["zero"], d["maxq"])
    rows = np.array([29, 3, 17])
    cs, Vs, Es = R.gptq_columns(d["W"], fa["P"], d["scale"], d["zero"], d["maxq"], rows=rows)
    assert np.array_equal(cs, c[rows]) and np.array_equal(Es, E[rows])


def test_special_case_A_identity_is_columnwise_gptq():
    d = make_problem(48, 20, 4, global_grid=True)
    fb = R.factor(d["B"])
    fa = R.factor(np.eye(20))
    c, _, _ = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    # columns of W are the rows of W^T; one global grid, so transposing is exact
    g = _textbook_gptq_rows(d["W"].T, fb["Ad"], d["scale"][:20], d["zero"][:20], d["maxq"][:20])
    assert np.array_equal(c, g.T)


def test_special_case_diagonal_factors_is_rounding():
    d = make_problem(17, 23, 5)
    rng = np.random.default_rng(5)
    fa = R.factor(np.diag(rng.uniform(0.5, 2.0, 23)))
    fb = R.factor(np.diag(rng.uniform(0.5, 2.0, 17)))
    c, V, _ = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    x = (d["W"] / d["scale"][:, None]).astype(np.float32) + d["zero"][:, None]
    rtn = np.clip(np.rint(x), 0, d["maxq"][:, None])
    assert np.array_equal(c, rtn)


def test_scaling_factors_leaves_codes():
    d = make_problem(24, 30, 6)
    fa, fb = _factors(d)
    fa2, fb2 = R.factor(d["A"] * 7.5), R.factor(d["B"] * 0.125)
    c1 = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])[0]
    c2 = R.bakron_naive(d["W"], fa2["P"], fb2["P"], d["scale"], d["zero"], d["maxq"])[0]
    assert np.array_equal(c1, c2)


def test_transpose_symmetry_global_grid():
    d = make_problem(19, 26, 7, global_grid=True)
    fa, fb = _factors(d)
    s, z, mq = d["scale"], d["zero"], d["maxq"]
    c1 = R.bakron_naive(d["W"], fa["P"], fb["P"], s, z, mq)[0]
    c2 = R.bakron_naive(d["W"].T, fb["P"], fa["P"], np.full(26, s[0]), np.full(26, z[0]),
                        np.full(26, mq[0]))[0]
    assert np.array_equal(c1, c2.T)


# The validator: passes every oracle output, and flags planted mistakes
# (planted in the oracle's output or arithmetic, on the CPU).
def test_validator_accepts_oracle_outputs():
    d = make_problem(96, 80, 8)
    fa, fb = _factors(d)
    c, V, E = O2.bakron_recursive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    r = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], fa["L"], fb["L"])
    assert r["mismatches"] == 0 and r["bad"] == 0


def test_validator_flags_planted_code_flip():
    d = make_problem(64, 64, 9)
    fa, fb = _factors(d)
    c, V, E = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    c = c.copy()
    i, j = 30, 41
    c[i, j] = c[i, j] + 1 if c[i, j] < d["maxq"][i] else c[i, j] - 1
    r = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], fa["L"], fb["L"])
    assert r["bad"] >= 1 and (i, j) in r["bad_index"]


@pytest.mark.parametrize("plant", ["drop_term", "sign", "transpose"])
def test_validator_flags_planted_arithmetic_mistake(plant):
    d = make_problem(48, 56, 10)
    fa, fb = _factors(d)
    PA, PB = fa["P"].copy(), fb["P"].copy()
    if plant == "drop_term":
        PA[30, 12] = 0.0
    elif plant == "sign":
        PB = 2 * np.eye(48) - PB            # flips the sign of every off-diagonal term
    else:
        PA = PA.T.copy()                    # transposed operand (upper triangular)
    c, V, E = R.bakron_naive(d["W"], PA, PB, d["scale"], d["zero"], d["maxq"])
    r = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], fa["L"], fb["L"])
    assert r["bad"] > 0


def test_validator_from_p_matches_from_l():
    d = make_problem(40, 72, 12)
    fa, fb = _factors(d)
    c, V, E = R.bakron_naive(d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    np.testing.assert_allclose(R.implied_errors_p(d["W"], V, fa["P"], fb["P"]), E, atol=1e-12)
    r = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], PA=fa["P"], PB=fb["P"])
    assert r["mismatches"] == 0


def test_validator_one_sided_identity_shortcut():
    # P_B omitted means B = I: the same implied errors and verdict as the
    # explicit identity
    d = make_problem(20, 36, 17)
    fa = R.factor(d["A"])
    c, V, E = R.gptq_columns(d["W"], fa["P"], d["scale"], d["zero"], d["maxq"])
    np.testing.assert_allclose(R.implied_errors_p(d["W"], V, fa["P"], None), E, atol=1e-12)
    a = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], PA=fa["P"], PB=None)
    b = R.validate(d["W"], c, d["scale"], d["zero"], d["maxq"], PA=fa["P"], PB=np.eye(20))
    assert a == b and a["mismatches"] == 0
    flip = c.copy()
    flip[7, 20] = flip[7, 20] + 1 if flip[7, 20] < d["maxq"][7] else flip[7, 20] - 1
    assert R.validate(d["W"], flip, d["scale"], d["zero"], d["maxq"], PA=fa["P"], PB=None)["bad"] >= 1


def test_dependency_cone_brute_force():
    """dependency_cone(mask)[i', j'] is true iff some masked (i, j) has
    i <= i' and j <= j' (checked entry by entry on random masks)."""
    rng = np.random.default_rng(3)
    for m, n, p in ((1, 1, 0.5), (5, 7, 0.05), (9, 4, 0.1), (6, 6, 0.0)):
        mask = rng.random((m, n)) < p
        c = R.dependency_cone(mask)
        for i in range(m):
            for j in range(n):
                assert c[i, j] == bool(mask[: i + 1, : j + 1].any())


# Tie-following mode of the C oracle (the comparison protocol for several
# valid outputs): following its own codes changes nothing; a code planted on
# the other side of the nearest-to-a-boundary decision is adopted when that
# decision lies within tau of the boundary, and a planted code away from any
# boundary is not.
def _margins(V, E, s, z, maxq):
    w = (V + E).astype(np.float32)
    x = (w / s[:, None].astype(np.float32)).astype(np.float32) + z[:, None].astype(np.float32)
    x = x.astype(np.float64)
    b = np.clip(np.floor(x) + 0.5, 0.5, maxq[:, None] - 0.5)
    return np.abs(x - b), x


def test_recursive_follow_mode():
    d = make_problem(48, 40, 23)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    args = (d["W"], fa["P"], fb["P"], d["scale"], d["zero"], d["maxq"])
    c, V, E = O2.bakron_recursive(*args, leaf=8)
    c2, V2, E2, k = O2.bakron_recursive(*args, leaf=8, follow=c, tau=0.5)
    assert k == 0 and np.array_equal(c2, c) and np.array_equal(E2, E)
    mg, x = _margins(V, E, d["scale"], d["zero"], d["maxq"])
    inner = (np.floor(x) >= 0) & (np.floor(x) < d["maxq"][:, None] - 1)   # both neighbours on the grid
    i, j = np.unravel_index(np.argmin(np.where(inner, mg, np.inf)), mg.shape)
    other = int(np.floor(x[i, j])) + (1 if c[i, j] == np.floor(x[i, j]) else 0)
    assert abs(other - c[i, j]) == 1
    plant = c.copy()
    plant[i, j] = other
    tau = 2 * mg[i, j] + 1e-12
    c3, V3, E3, k3 = O2.bakron_recursive(*args, leaf=8, follow=plant, tau=tau)
    assert c3[i, j] == other and k3 >= 1
    v = R.validate(d["W"], c3, d["scale"], d["zero"], d["maxq"], tau=tau, PA=fa["P"], PB=fb["P"])
    assert v["bad"] == 0 and v["ties"] >= 1
    # a plant far from any boundary is ignored
    i2, j2 = np.unravel_index(np.argmax(np.where(inner, mg, -1)), mg.shape)
    plant2 = c.copy()
    plant2[i2, j2] = c[i2, j2] + (1 if c[i2, j2] < d["maxq"][i2] else -1)
    c4, _, _, k4 = O2.bakron_recursive(*args, leaf=8, follow=plant2, tau=1e-4)
    assert k4 == 0 and np.array_equal(c4, c)


def test_gptq_columns_follow_mode():
    d = make_problem(30, 50, 16)
    fa = R.factor(d["A"])
    args = (d["W"], fa["P"], d["scale"], d["zero"], d["maxq"])
    c, V, E = R.gptq_columns(*args)
    c2, _, _, k = R.gptq_columns(*args, follow=c, tau=0.5)
    assert k == 0 and np.array_equal(c2, c)
    mg, x = _margins(V, E, d["scale"], d["zero"], d["maxq"])
    inner = (np.floor(x) >= 0) & (np.floor(x) < d["maxq"][:, None] - 1)
    i, j = np.unravel_index(np.argmin(np.where(inner, mg, np.inf)), mg.shape)
    other = int(np.floor(x[i, j])) + (1 if c[i, j] == np.floor(x[i, j]) else 0)
    plant = c.copy()
    plant[i, j] = other
    c3, _, _, k3 = R.gptq_columns(*args, follow=plant, tau=2 * mg[i, j] + 1e-12)
    assert c3[i, j] == other and k3 >= 1
    # the adopted flip only changes row i (rows are independent)
    same = np.ones(c.shape[0], bool)
    same[i] = False
    assert np.array_equal(c3[same], c[same])
