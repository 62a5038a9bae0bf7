"""Float64 reference forms of the BaKron solve (TEST INFRASTRUCTURE ONLY).

Only tests, the smoke check and the bench CPU baseline may use this module.

Notation (from [S], setup paragraph and Corollary 3.4): W is m x n, row i is
an output coordinate and column j an input coordinate.  The Hessian of the
layer loss is approximated by A (x) B with A (n x n) on the input side and
B (m x m) on the output side, so that for Delta = V - W the loss proxy is
vec(Delta)^T (A (x) B) vec(Delta) = ||B^(1/2) Delta A^(1/2)||_F^2 with the
column-major vec.  GPTQ is the special case B = I ([S] setup; [N5]).

Readings taken where the pages are silent (each is listed in the design doc):

* Damping: A_d = A + frac * mean(diag A) * I, frac = 0.01, and the same for
  B.  The pages do not mention damping; this is the usual GPTQ convention.
* RevCholesky(A) ([S] Corollary 3.4) is the lower-triangular L with
  A = L^T L.  It is the only reading under which ||L(B)(V-W)L(A)^T||_F^2
  equals the A (x) B loss.
* Processing order: GPTQ on vec(W) in column-major order ([S], BaKron-naive),
  equivalently any order that visits (i, j) after every (i', j') with
  i' <= i and j' <= j ([S], BaKron-antidiagonal: an entry's update only
  reaches entries below and to the right of it; Theorem 3.2).
* The base quantizer is modular ([A]); here it is a uniform grid per output
  row: x = w/s_i + z_i, code c = clamp(rint(x), 0, maxq_i) with
  round-half-to-even, value v = s_i (c - z_i).  The rounding decision is
  taken in float32 (x formed as float32(float32(w) / s) + z in float32), the
  precision of the kernels, so that both sides decide in the same
  precision.  Everything else here is float64.
* A clipped entry keeps its full error (GPTQ convention).
* Per-group grids (the base quantizer is modular, [A]): with a group size g,
  entry (i, j) is rounded on the grid (s, z, maxq)[i, j // g] -- static
  groups along the input dimension, each grid a fixed input (computed by the
  caller from the original W).  A grid that depended on the working weights
  at the group's first column would depend on the order the entries are
  visited in, and the forms below (Theorem 3.2) would no longer agree.
  Every form takes the grid either per output row (1-D arrays, group_size
  None) or per (row, group) (m x G arrays, G = ceil(n / group_size)).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "damp", "rev_cholesky", "normalized_inverse", "factor", "factor_float32", "quantize",
    "gptq_vectorized", "bakron_naive", "bakron_antidiagonal", "bakron_lform", "gptq_columns",
    "kron_moment", "row_sqnorms", "kfac_factors", "shampoo_factors",
    "objective", "objective_from_errors", "implied_errors", "implied_errors_p", "validate", "entry_grid",
    "order_colmajor", "order_rowmajor", "order_antidiagonal",
]

_f32 = np.float32


# ------------------------------------------- Kronecker factors from samples

def row_sqnorms(X) -> np.ndarray:
    """|x_t|^2 for every row x_t of the sample-major matrix X (float64)."""
    X = np.asarray(X, np.float64)
    return np.sum(X * X, axis=1)


def kron_moment(X, w=None, scale=None) -> np.ndarray:
    """M = scale * sum_t w_t x_t x_t^T, x_t = row t of X, in float64
    (scale defaults to 1 / N: an expectation over the samples)."""
    X = np.asarray(X, np.float64)
    N = X.shape[0]
    if scale is None:
        scale = 1.0 / N
    Xw = X if w is None else X * np.asarray(w, np.float64)[:, None]
    return scale * (Xw.T @ X)


def kfac_factors(Xa, Xb):
    """K-FAC-style independence ([S], Hessian choices): the Hessian of the
    layer, E[(a (x) b)(a (x) b)^T] = E[a a^T (x) b b^T], is replaced by
    E[a a^T] (x) E[b b^T].  Xa (N x n) holds the input activations a_t,
    Xb (N x m) the output gradients b_t, one sample per row."""
    return kron_moment(Xa), kron_moment(Xb)


def shampoo_factors(Xa, Xb):
    """Shampoo-style ([S], Hessian choices): one power-iteration step of the
    nearest Kronecker product A (x) B to E[a a^T (x) b b^T], started from the
    identity on the other side, gives A = E[|b|^2 a a^T] and
    B = E[|a|^2 b b^T]."""
    return kron_moment(Xa, row_sqnorms(Xb)), kron_moment(Xb, row_sqnorms(Xa))


# ---------------------------------------------------------------- factor step

def damp(A: np.ndarray, frac: float = 0.01) -> np.ndarray:
    """A + frac * mean(diag(A)) * I in float64 (damping reading, see header)."""
    A = np.asarray(A, dtype=np.float64)
    A = 0.5 * (A + A.T)
    return A + frac * np.mean(np.diag(A)) * np.eye(A.shape[0])


def rev_cholesky(Ad: np.ndarray) -> np.ndarray:
    """RevCholesky ([S] Corollary 3.4): lower L with Ad = L^T L.

    Written as the flip of the textbook Cholesky: with J the exchange matrix,
    J Ad J = C C^T (C lower); then L = J C^T J is lower triangular and
    L^T L = J C C^T J = Ad.
    Raises numpy.linalg.LinAlgError when Ad is not positive definite.
    """
    Ad = np.asarray(Ad, dtype=np.float64)
    C = np.linalg.cholesky(Ad[::-1, ::-1])
    return np.ascontiguousarray(C.T[::-1, ::-1])


def normalized_inverse(L: np.ndarray) -> np.ndarray:
    """P = L^-1 diag(L): unit lower triangular.

    Derived from [S] (GPTQ on vec(W) with Hessian A (x) B): with Ad = L^T L,
    the upper Cholesky factor of Ad^-1 is L^-T, so GPTQ's normalised update
    row for index j is column j of L^-1 scaled by L_jj, i.e. column j of P.
    """
    L = np.asarray(L, dtype=np.float64)
    n = L.shape[0]
    Li = np.linalg.solve(L, np.eye(n))        # library triangular-capable solve
    Li = np.tril(Li)
    return Li * np.diag(L)[None, :]


def factor(A: np.ndarray, frac: float = 0.01) -> dict:
    """Damping, RevCholesky and the normalised inverse of one Kronecker factor."""
    Ad = damp(A, frac)
    L = rev_cholesky(Ad)
    return {"Ad": Ad, "L": L, "P": normalized_inverse(L)}


def factor_float32(A: np.ndarray, frac: float = 0.01) -> dict:
    """The same factor step carried out in float32 arithmetic by the
    library routines (LAPACK's single-precision Cholesky and triangular
    solve): a float32 factorisation independent of the HIP path, whose
    rounding errors (about n u cond(A_d)) are of the kind a float32 solver's
    factors carry.  Used only to measure how far two valid float32 runs can
    land from the float64 one (tests/golden/trajectory_spread.py)."""
    from scipy.linalg import solve_triangular
    A = np.asarray(A, dtype=np.float32)
    n = A.shape[0]
    A = ((A + A.T) * np.float32(0.5)).astype(np.float32)
    add = np.float32(frac) * np.float32(np.mean(np.diag(A).astype(np.float64)))
    Ad = A + add * np.eye(n, dtype=np.float32)
    C = np.linalg.cholesky(Ad[::-1, ::-1])              # float32 in, float32 factor
    L = np.ascontiguousarray(C.T[::-1, ::-1])
    Li = solve_triangular(L, np.eye(n, dtype=np.float32), lower=True)
    P = (np.tril(Li) * np.diag(L)[None, :]).astype(np.float32)
    return {"Ad": Ad, "L": L, "P": P}


# ------------------------------------------------------------ base quantizer

def quantize(w, s, z, maxq):
    """Uniform grid of one output row: returns (code, value).

    The decision x = w/s + z is formed in float32 (the kernels' precision);
    the value s (c - z) is returned in float64.  Works elementwise on arrays.
    """
    x = (np.asarray(w, dtype=np.float64).astype(_f32) / np.asarray(s, dtype=_f32)).astype(_f32) \
        + np.asarray(z, dtype=_f32)
    x = np.asarray(x, dtype=_f32)
    c = np.minimum(np.maximum(np.rint(x), _f32(0)), np.asarray(maxq).astype(_f32))
    c = c.astype(np.float64)
    v = np.asarray(s, dtype=np.float64) * (c - np.asarray(z, dtype=np.float64))
    return c, v


def entry_grid(s, z, maxq, m, n, group_size=None):
    """The grid of every entry as three m x n arrays: (s, z, maxq)[i] for a
    per-row grid (1-D inputs, group_size None), (s, z, maxq)[i, j // g] for
    per-group grids (m x G inputs, group_size g)."""
    s, z, maxq = np.asarray(s), np.asarray(z), np.asarray(maxq)
    if group_size is None:
        if s.ndim != 1:
            raise ValueError("per-row grids are 1-D; pass group_size with m x G grids")
        cols = np.zeros(n, dtype=np.int64)
        s, z, maxq = s[:, None], z[:, None], maxq[:, None]
    else:
        g = int(group_size)
        G = -(-n // g) if n else 0
        if s.shape != (m, G) or z.shape != (m, G) or maxq.shape != (m, G):
            raise ValueError(f"per-group grids must be {m} x {G}")
        cols = np.arange(n) // g
    return (np.ascontiguousarray(s[:, cols]), np.ascontiguousarray(z[:, cols]),
            np.ascontiguousarray(maxq[:, cols]))


def _values(codes, s, z, group_size=None):
    codes = np.asarray(codes, np.float64)
    S, Z, _ = entry_grid(s, z, np.zeros(np.shape(s), np.int32), *codes.shape, group_size)
    return S.astype(np.float64) * (codes - Z.astype(np.float64))


# --------------------------------------------------- O1a: brute force on vec(W)

def gptq_vectorized(W, Ad, Bd, s, z, maxq, group_size=None):
    """GPTQ run directly on vec(W) with the explicit Hessian H = Ad (x) Bd.

    This is the definition BaKron-naive starts from ([S], derivation: GPTQ in
    the vectorised domain with Hessian A (x) B).  Column-major vec: index
    p = j*m + i, and numpy.kron(Ad, Bd)[(j,i),(j',i')] = Ad[j,j'] Bd[i,i'].
    GPTQ step (textbook): with H^-1 = U^T U (U upper), quantize w_p, then
    w_q -= (w_p - v_p) / U_pp * U_pq for q > p.  Only for m*n <= 4096.
    Returns (codes, V) as m x n arrays.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    if m * n > 4096:
        raise ValueError("brute force is limited to m*n <= 4096")
    S, Z, Q = entry_grid(s, z, maxq, m, n, group_size)
    H = np.kron(np.asarray(Ad, np.float64), np.asarray(Bd, np.float64))
    Hinv = np.linalg.inv(H)
    Hinv = 0.5 * (Hinv + Hinv.T)
    U = np.linalg.cholesky(Hinv).T            # upper, Hinv = U^T U
    w = W.flatten(order="F").copy()
    codes = np.zeros(m * n)
    vals = np.zeros(m * n)
    for p in range(m * n):
        i, j = p % m, p // m
        c, v = quantize(w[p], S[i, j], Z[i, j], Q[i, j])
        codes[p], vals[p] = c, v
        err = (w[p] - v) / U[p, p]
        w[p:] -= err * U[p, p:]
    return codes.reshape((m, n), order="F"), vals.reshape((m, n), order="F")


# ------------------------------------------------ O1b: BaKron-naive, any order

def order_colmajor(m, n):
    return [(i, j) for j in range(n) for i in range(m)]


def order_rowmajor(m, n):
    return [(i, j) for i in range(m) for j in range(n)]


def order_antidiagonal(m, n):
    return [(i, k - i) for k in range(m + n - 1) for i in range(max(0, k - n + 1), min(m - 1, k) + 1)]


def bakron_naive(W, PA, PB, s, z, maxq, order=None, group_size=None):
    """BaKron-naive in the matrix domain ([S], derivation, first variant).

    One entry at a time; after quantizing (i, j) with raw error e, every entry
    to its bottom-right receives W~[i', j'] -= e * PB[i', i] * PA[j', j]
    (Proposition 3.1 turns the vec-domain rank-1 GPTQ update into this outer
    product).  ``order`` is any linear extension of the bottom-right partial
    order (Theorem 3.2); default column-major.
    Returns (codes, V, E) with E the raw errors w~ - v.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    PA = np.asarray(PA, np.float64)
    PB = np.asarray(PB, np.float64)
    S, Z, Q = entry_grid(s, z, maxq, m, n, group_size)
    Wt = W.copy()
    C = np.zeros((m, n))
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    for (i, j) in (order if order is not None else order_colmajor(m, n)):
        c, v = quantize(Wt[i, j], S[i, j], Z[i, j], Q[i, j])
        e = Wt[i, j] - v
        C[i, j], V[i, j], E[i, j] = c, v, e
        Wt[i:, j:] -= e * np.outer(PB[i:, i], PA[j:, j])
    return C, V, E


# ------------------------------------- one-sided case B = I (GPTQ), by column

def gptq_columns(W, PA, s, z, maxq, rows=None, follow=None, tau=1e-4, group_size=None):
    """The one-sided case B = I of the rounding ([S] setup: GPTQ's Hessian is
    A (x) I; [N5]).  With P_B = I the update of BaKron-naive,
    W~[i', j'] -= e P_B[i', i] P_A[j', j], only reaches later columns of the
    same row, so every row is rounded column by column independently:
    for j = 0 .. n-1, round column j of all rows, then
    W~[:, j'] -= e P_A[j', j] for j' > j.
    ``rows`` selects a subset of the rows (each row depends on nothing else).
    ``follow`` (codes of another implementation, for the selected rows) turns
    on tie following as in recursive.c: where the float32 decision lies
    within ``tau`` grid steps of a rounding boundary and the followed code is
    the neighbouring one, it is taken over.
    Returns (codes, V, E) for the selected rows, and with ``follow`` also the
    number of codes taken over.
    """
    W = np.asarray(W, dtype=np.float64)
    PA = np.asarray(PA, np.float64)
    S, Z, Q = entry_grid(s, z, maxq, W.shape[0], W.shape[1], group_size)
    if rows is not None:
        rows = np.asarray(rows)
        W, S, Z, Q = W[rows], S[rows], Z[rows], Q[rows]
    m, n = W.shape
    Wt = W.copy()
    C = np.zeros((m, n))
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    adopted = 0
    for j in range(n):
        s, z, maxq = S[:, j], Z[:, j], Q[:, j]
        c, v = quantize(Wt[:, j], s, z, maxq)
        if follow is not None:
            x = (Wt[:, j].astype(_f32) / s.astype(_f32)).astype(_f32) + z.astype(_f32)
            x = x.astype(np.float64)
            bnd = np.clip(np.floor(x) + 0.5, 0.5, maxq - 0.5)
            g = np.asarray(follow)[:, j].astype(np.float64)
            take = (np.abs(g - c) == 1) & (np.abs(x - bnd) < tau)
            if take.any():
                c = np.where(take, g, c)
                v = s.astype(np.float64) * (c - z.astype(np.float64))
                adopted += int(take.sum())
        e = Wt[:, j] - v
        C[:, j], V[:, j], E[:, j] = c, v, e
        Wt[:, j + 1:] -= np.outer(e, PA[j + 1:, j])
    if follow is not None:
        return C, V, E, adopted
    return C, V, E


# ------------------------------------------------ O1c: BaKron-antidiagonal

def bakron_antidiagonal(W, PA, PB, s, z, maxq, group_size=None):
    """BaKron-antidiagonal ([S], derivation, second variant).

    All entries with i + j = k are quantized together (they do not update one
    another), then their errors are pushed to the rest of the matrix at once:
    W~ -= PB E_k PA^T, where E_k holds the raw errors of anti-diagonal k.
    Because PB and PA are lower triangular this only touches entries below
    and to the right of each source; the self term leaves w~_ij = v_ij.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    PA = np.asarray(PA, np.float64)
    PB = np.asarray(PB, np.float64)
    S, Z, Q = entry_grid(s, z, maxq, m, n, group_size)
    Wt = W.copy()
    C = np.zeros((m, n))
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    for k in range(m + n - 1):
        ii = np.arange(max(0, k - n + 1), min(m - 1, k) + 1)
        jj = k - ii
        c, v = quantize(Wt[ii, jj], S[ii, jj], Z[ii, jj], Q[ii, jj])
        e = Wt[ii, jj] - v
        C[ii, jj], V[ii, jj], E[ii, jj] = c, v, e
        Ek = np.zeros((m, n))
        Ek[ii, jj] = e
        Wt -= PB @ Ek @ PA.T
    return C, V, E


# ------------------------------------------------ O1d: inverse-free L-form

def bakron_lform(W, LA, LB, s, z, maxq, order=None, group_size=None):
    """The same rounding written with L(A), L(B) only (no inverse).

    From W - V = PB E PA^T and PB^-1 = diag(LB)^-1 LB (likewise for A), the
    value an entry is rounded from is
      w~_ij = W_ij + sum over strict predecessors (i', j') of
              LB[i, i'] LA[j, j'] (W - V)_{i'j'} / (LB_ii LA_jj),
    i.e. a nearest-plane recursion in the L(B) (x) L(A) lattice basis
    ([S] Corollary 3.4 uses the same factors).  ``order`` as in bakron_naive.
    """
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    LA = np.asarray(LA, np.float64)
    LB = np.asarray(LB, np.float64)
    S, Z, Q = entry_grid(s, z, maxq, m, n, group_size)
    D = np.zeros((m, n))          # (W - V) on processed entries, 0 elsewhere
    C = np.zeros((m, n))
    V = np.zeros((m, n))
    E = np.zeros((m, n))
    for (i, j) in (order if order is not None else order_colmajor(m, n)):
        acc = LB[i, : i + 1] @ D[: i + 1, : j + 1] @ LA[j, : j + 1]
        wt = W[i, j] + acc / (LB[i, i] * LA[j, j])
        c, v = quantize(wt, S[i, j], Z[i, j], Q[i, j])
        C[i, j], V[i, j], E[i, j] = c, v, wt - v
        D[i, j] = W[i, j] - v
    return C, V, E


# ----------------------------------------------------------------- objective

def objective(W, V, LA, LB) -> float:
    """||L(B) (V - W) L(A)^T||_F^2 ([S] Corollary 3.4), in float64."""
    D = np.asarray(V, np.float64) - np.asarray(W, np.float64)
    M = np.asarray(LB, np.float64) @ D @ np.asarray(LA, np.float64).T
    return float(np.sum(M * M))


def objective_from_errors(E, LA, LB) -> float:
    """sum_ij (LB_ii LA_jj e_ij)^2; equals ``objective`` because
    L(B)(W - V)L(A)^T = diag(LB) E diag(LA) (derived from W - V = PB E PA^T)."""
    M = np.diag(np.asarray(LB, np.float64))[:, None] * np.asarray(E, np.float64) \
        * np.diag(np.asarray(LA, np.float64))[None, :]
    return float(np.sum(M * M))


def implied_errors(W, V, LA, LB) -> np.ndarray:
    """The raw errors E that any run producing V must have had.

    Inverts W - V = PB E PA^T: E = diag(LB)^-1 LB (W - V) LA^T diag(LA)^-1.
    """
    D = np.asarray(W, np.float64) - np.asarray(V, np.float64)
    M = np.asarray(LB, np.float64) @ D @ np.asarray(LA, np.float64).T
    return M / (np.diag(LB)[:, None] * np.diag(LA)[None, :])


def implied_errors_p(W, V, PA, PB) -> np.ndarray:
    """Same as ``implied_errors`` but from P_A, P_B directly:
    E = PB^-1 (W - V) PA^-T by two unit-lower triangular solves.
    PB None stands for the identity (the one-sided case B = I)."""
    from scipy.linalg import solve_triangular
    D = np.asarray(W, np.float64) - np.asarray(V, np.float64)
    if PB is None:
        X = D
    else:
        X = solve_triangular(np.asarray(PB, np.float64), D, lower=True, unit_diagonal=True)
    Et = solve_triangular(np.asarray(PA, np.float64), X.T, lower=True, unit_diagonal=True)
    return np.ascontiguousarray(Et.T)


# ----------------------------------------------------------------- validator

def validate(W, codes, s, z, maxq, LA=None, LB=None, tau=1e-4, PA=None, PB=None,
             return_errors=False, group_size=None) -> dict:
    """Check that ``codes`` is a BaKron output for (W, A (x) B, grid), any size.

    For a sequence of rounding decisions, the value entry (i, j) is rounded
    from is w~_ij = v_ij + e_ij with E = ``implied_errors`` (it depends only
    on decisions that precede (i, j)).  A valid output has, at every entry,
    code == clamp(rint(w~/s + z)).  Near a rounding boundary float32 and
    float64 may legitimately disagree (Theorem 3.2's equality is exact only
    in exact arithmetic), so a mismatch is a "tie" when x lies within
    ``tau`` grid steps of the boundary and the codes are adjacent.

    The factors are given either as L_A, L_B or as P_A, P_B (P_B None: the
    identity, i.e. the one-sided case B = I).
    Returns counts: entries, mismatches, ties (allowed), bad (outside the
    tie band or more than one step apart), max_step, min_margin; with
    ``return_errors`` also the implied errors as "E" and the boolean masks
    "tie_mask" and "bad_mask".
    """
    W = np.asarray(W, np.float64)
    m, n = W.shape
    codes = np.asarray(codes, np.float64)
    ss, zz, mq = entry_grid(s, z, maxq, m, n, group_size)
    V = ss.astype(np.float64) * (codes - zz.astype(np.float64))
    if PA is not None:
        E = implied_errors_p(W, V, PA, PB)
    else:
        E = implied_errors(W, V, LA, LB)
    Wt = V + E
    cexp, _ = quantize(Wt, ss, zz, mq)
    x = (Wt.astype(_f32) / ss.astype(_f32)).astype(_f32) + zz.astype(_f32)
    x = x.astype(np.float64)
    bnd = np.clip(np.floor(x) + 0.5, 0.5, mq - 0.5)
    margin = np.abs(x - bnd)
    diff = codes - cexp
    mism = diff != 0
    ties = mism & (margin < tau) & (np.abs(diff) == 1)
    bad = mism & ~ties
    out = {
        "entries": int(m * n),
        "mismatches": int(mism.sum()),
        "ties": int(ties.sum()),
        "bad": int(bad.sum()),
        "max_step": int(np.abs(diff).max()) if m * n else 0,
        "min_margin": float(margin.min()) if m * n else float("inf"),
        "bad_index": [tuple(map(int, t)) for t in np.argwhere(bad)[:8]],
    }
    if return_errors:
        out["E"] = E
        out["tie_mask"] = ties
        out["bad_mask"] = bad
    return out


def dependency_cone(mask) -> np.ndarray:
    """Entries (i', j') with some masked (i, j), i <= i' and j <= j': the
    entries whose rounded-from value depends on a masked decision ([S]
    derivation: entry (i, j) only updates entries to its bottom-right)."""
    c = np.logical_or.accumulate(np.asarray(mask, bool), axis=0)
    return np.logical_or.accumulate(c, axis=1)
