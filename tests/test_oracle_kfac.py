"""Pins of the oracle's Kronecker-factor construction (CPU).

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians", Hessian choices (K-FAC-style independence;
Shampoo-style power iteration from the identity).

The readings are checked against the per-sample Hessian written out in full
on tiny shapes: H = E[(a (x) b)(a (x) b)^T] over column-major vec(W), the
Van Loan-Pitsianis rearrangement R(H) (whose best rank-one approximation
gives the nearest Kronecker product) and one power-iteration step from the
identity, all by explicit index loops.
"""
import numpy as np

from oracle import reference as R


def _explicit_hessian(Xa, Xb):
    N, n = Xa.shape
    m = Xb.shape[1]
    H = np.zeros((n * m, n * m))
    for t in range(N):
        g = np.zeros(n * m)          # vec of the per-sample gradient b a^T (m x n), column-major
        for j in range(n):
            for i in range(m):
                g[j * m + i] = Xb[t, i] * Xa[t, j]
        H += np.outer(g, g)
    return H / N


def test_shampoo_is_one_power_step_of_nearest_kronecker_product():
    rng = np.random.default_rng(0)
    N, n, m = 7, 4, 3
    Xa, Xb = rng.standard_normal((N, n)), rng.standard_normal((N, m))
    H = _explicit_hessian(Xa, Xb)
    # R(H)[(j, j'), (i, i')] = H[j m + i, j' m + i'];  A1 = R(H) vec(I_m),  B1 = R(H)^T vec(I_n)
    A1 = np.zeros((n, n))
    B1 = np.zeros((m, m))
    for j in range(n):
        for jp in range(n):
            A1[j, jp] = sum(H[j * m + i, jp * m + i] for i in range(m))
    for i in range(m):
        for ip in range(m):
            B1[i, ip] = sum(H[j * m + i, j * m + ip] for j in range(n))
    A, B = R.shampoo_factors(Xa, Xb)
    np.testing.assert_allclose(A, A1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(B, B1, rtol=1e-12, atol=1e-12)


def test_kfac_is_exact_when_the_gradient_is_constant():
    # b_t = b0 for every sample: H = E[a a^T] (x) b0 b0^T exactly
    rng = np.random.default_rng(1)
    N, n, m = 6, 3, 4
    Xa = rng.standard_normal((N, n))
    b0 = rng.standard_normal(m)
    Xb = np.tile(b0, (N, 1))
    H = _explicit_hessian(Xa, Xb)
    A, B = R.kfac_factors(Xa, Xb)
    np.testing.assert_allclose(np.kron(A, B), H, rtol=1e-12, atol=1e-12)


def test_moment_of_one_hot_samples_is_the_histogram():
    # x_t = e_{k(t)}: E[x x^T] = diag(counts) / N
    k = np.array([0, 2, 2, 3, 0, 2, 1, 1, 2])
    X = np.eye(5)[k]
    M = R.kron_moment(X)
    np.testing.assert_array_equal(M, np.diag(np.bincount(k, minlength=5) / len(k)))


def test_weighted_moment_and_norms_invariants():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((50, 12))
    w = rng.random(50)
    M = R.kron_moment(X, w, scale=1.0)
    assert np.allclose(M, M.T)
    assert np.linalg.eigvalsh(M).min() > 0             # positive weights, full column rank
    # trace(sum_t w_t x_t x_t^T) = sum_t w_t |x_t|^2
    assert np.isclose(np.trace(M), np.dot(w, R.row_sqnorms(X)), rtol=1e-12)
    # scaling a sample's weight by c scales its rank-one term: moving the
    # weight into the sample (x_t -> sqrt(w_t) x_t) gives the same moment
    np.testing.assert_allclose(R.kron_moment(X * np.sqrt(w)[:, None], scale=1.0), M, rtol=1e-12, atol=1e-12)
