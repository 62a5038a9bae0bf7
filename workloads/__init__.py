"""Seeded synthetic workloads for the BaKron solve.

This module only draws inputs; it holds none of the solver's arithmetic.  Both
the test oracle and the HIP path consume what it produces, so neither has to
import the other.

A workload is a weight W (m x n, output rows i, input columns j), two
Kronecker factors A (n x n, input side) and B (m x m, output side) of the
Hessian A (x) B, and a base quantizer grid per output row.  The pages on
BaKron ("BaKron: Efficient Quantization with Kronecker-Factored Hessians",
paper summary, setup paragraph) leave the base quantizer open ("modular");
the grid used here is a per-row asymmetric min-max uniform grid computed
from the original row of W.

Recipe (all draws in float64 from ``numpy.random.default_rng(seed)``, in
this fixed order: W; then the X channel scales and X; then the G channel
scales and G; then, for mixed precision, the row permutation):

* A = X X^T / N and B = G G^T / N, undamped (damping belongs to the factor
  step).  X is n x N, G is m x N.
* "log-normal channel scales": row k of X (or G) is multiplied by exp(xi_k),
  xi_k ~ N(0, 1), which produces outlier channels.
* Grid of row i: s_i = (max_j W_ij - min_j W_ij) / maxq_i and
  z_i = -min_j W_ij / s_i (fractional zero point), computed in float64 and
  then rounded to float32; both sides use those float32 values.
* Per-group grids (``group_size`` g): the same min-max rule on each row's
  slice of g columns of the original W (static groups; the last group may
  be shorter), giving m x ceil(n / g) arrays; every group of a row keeps
  the row's maxq.
* W, A, B are rounded to float32 at the end.

The named configurations stand in for the transformer layers that the pages
evaluate on (Llama / Qwen linear layers); no model weights or calibration
data are used.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

__all__ = ["Spec", "CONFIGS", "by_name", "generate", "samples", "make_problem", "grid_minmax", "grid_groups",
           "digest"]


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    m: int
    n: int
    w_dist: str            # "normal" or "student5"
    w_scale: float
    samples: int           # N: columns of X and of G
    lognormal: bool        # log-normal(sigma=1) channel scales on X and G
    bits: int              # uniform bit width (maxq = 2**bits - 1) ...
    mixed_low_rows: int = 0  # ... except this many rows (random) get bits-1
    seed: int = 0

    @property
    def shape(self):
        return (self.m, self.n)


# The five workload families (six shapes).  The 4096 x 14336 pair mimics the
# up/down projections of a GLU MLP; the 8192^2 mixed 2/3-bit case averages
# (1638*2 + 6554*3)/8192 = 2.80005 bits per weight.
CONFIGS = [
    Spec("tiny64", 64, 64, "normal", 0.02, 512, False, 4),
    Spec("sq1024", 1024, 1024, "normal", 0.02, 2048, True, 3),
    Spec("sq4096_t5", 4096, 4096, "student5", 0.02, 4096, True, 2),
    Spec("glu_up_4096x14336", 4096, 14336, "normal", 0.02, 4096, True, 3),
    Spec("glu_down_14336x4096", 14336, 4096, "normal", 0.02, 4096, True, 3),
    Spec("sq8192_mixed", 8192, 8192, "normal", 0.015, 8192, True, 3, mixed_low_rows=1638),
]


def by_name(name: str) -> Spec:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(name)


def grid_minmax(W: np.ndarray, maxq: np.ndarray):
    """Per-output-row asymmetric min-max uniform grid (float64 -> float32)."""
    W = np.asarray(W, dtype=np.float64)
    lo = W.min(axis=1)
    hi = W.max(axis=1)
    mq = np.asarray(maxq, dtype=np.float64)
    s = (hi - lo) / mq
    if np.any(s <= 0):
        raise ValueError("degenerate row (max == min): the grid would have zero step")
    z = -lo / s
    return s.astype(np.float32), z.astype(np.float32)


def grid_groups(W: np.ndarray, maxq: np.ndarray, group_size: int):
    """Asymmetric min-max grids per (row, group of group_size columns) of the
    original W: scale, zero (float32) and maxq (int32), each m x G."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    g = int(group_size)
    if g < 1:
        raise ValueError("group_size must be positive")
    G = -(-n // g)
    s = np.empty((m, G), np.float32)
    z = np.empty((m, G), np.float32)
    for k in range(G):
        s[:, k], z[:, k] = grid_minmax(W[:, k * g:(k + 1) * g], maxq)
    return s, z, np.repeat(np.asarray(maxq, np.int32)[:, None], G, axis=1)


def _draw_samples(rng, dim, samples, lognormal):
    """dim x samples draws (feature-major), with log-normal channel scales."""
    if lognormal:
        sc = np.exp(rng.standard_normal(dim))
    X = rng.standard_normal((dim, samples))
    if lognormal:
        X *= sc[:, None]
    return X


def _draw_w(rng, spec):
    m, n = spec.m, spec.n
    if spec.w_dist == "normal":
        return rng.standard_normal((m, n)) * spec.w_scale
    if spec.w_dist == "student5":
        return rng.standard_t(5, size=(m, n)) * spec.w_scale
    raise ValueError(spec.w_dist)


def generate(spec: Spec, seed: int | None = None, global_grid: bool = False, group_size: int | None = None) -> dict:
    """Draw one workload; returns float32 W, A, B, scale, zero and int32 maxq.

    ``global_grid`` replaces the per-row grid by one grid for the whole
    matrix (same step and zero point on every row; needed when n == 1).
    ``group_size`` gives per-group grids (scale, zero, maxq m x G) instead."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    m, n = spec.m, spec.n
    W = _draw_w(rng, spec)
    X = _draw_samples(rng, n, spec.samples, spec.lognormal)
    A = X @ X.T / spec.samples
    del X
    G = _draw_samples(rng, m, spec.samples, spec.lognormal)
    B = G @ G.T / spec.samples
    del G
    maxq = np.full(m, 2 ** spec.bits - 1, dtype=np.int32)
    if spec.mixed_low_rows:
        rows = rng.permutation(m)[: spec.mixed_low_rows]
        maxq[rows] = 2 ** (spec.bits - 1) - 1
    W32 = W.astype(np.float32)
    if group_size is not None:
        s, z, maxq = grid_groups(W32, maxq, group_size)
    elif global_grid:
        s, z = grid_minmax(W32.reshape(1, -1), maxq[:1])
        s = np.full(m, s[0], dtype=np.float32)
        z = np.full(m, z[0], dtype=np.float32)
    else:
        s, z = grid_minmax(W32, maxq)
    return {
        "W": W32,
        "A": A.astype(np.float32),
        "B": B.astype(np.float32),
        "scale": s,
        "zero": z,
        "maxq": maxq,
        "name": spec.name,
    }


def samples(spec: Spec, seed: int | None = None) -> dict:
    """The per-sample inputs behind A and B of ``generate`` (same draws):
    X (N x n) input activations and G (N x m) output gradients, sample-major
    (row t is sample t), float32.  ``generate`` forms A = X^T X / N and
    B = G^T G / N from the float64 draws; these are the float32 samples."""
    rng = np.random.default_rng(spec.seed if seed is None else seed)
    _draw_w(rng, spec)
    X = _draw_samples(rng, spec.n, spec.samples, spec.lognormal)
    Xs = np.ascontiguousarray(X.T, dtype=np.float32)
    del X
    G = _draw_samples(rng, spec.m, spec.samples, spec.lognormal)
    Gs = np.ascontiguousarray(G.T, dtype=np.float32)
    return {"X": Xs, "G": Gs, "name": spec.name}


def make_problem(m: int, n: int, seed: int, bits: int = 3, samples: int | None = None,
                 lognormal: bool = True, w_scale: float = 0.02, global_grid: bool = False,
                 group_size: int | None = None) -> dict:
    """A small workload with the same recipe at an arbitrary shape (tests)."""
    spec = Spec(f"p{m}x{n}s{seed}", m, n, "normal", w_scale,
                samples if samples is not None else 2 * max(m, n), lognormal, bits, seed=seed)
    return generate(spec, global_grid=global_grid, group_size=group_size)


def digest(d: dict) -> str:
    """Stable hash of a workload's arrays (determinism checks)."""
    h = hashlib.sha256()
    for k in ("W", "A", "B", "scale", "zero", "maxq"):
        a = np.ascontiguousarray(d[k])
        h.update(k.encode())
        h.update(str(a.dtype).encode())
        h.update(str(a.shape).encode())
        h.update(a.tobytes())
    return h.hexdigest()
