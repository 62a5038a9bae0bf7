"""The seeded generators: determinism and the recipe's stated properties."""
import numpy as np

import workloads as WL


def test_deterministic_and_seed_sensitive():
    a = WL.make_problem(40, 24, 3)
    b = WL.make_problem(40, 24, 3)
    c = WL.make_problem(40, 24, 4)
    assert WL.digest(a) == WL.digest(b)
    assert WL.digest(a) != WL.digest(c)


def test_config_table():
    names = [c.name for c in WL.CONFIGS]
    assert len(names) == len(set(names)) == 6
    shapes = {c.name: c.shape for c in WL.CONFIGS}
    assert shapes["tiny64"] == (64, 64)
    assert shapes["sq8192_mixed"] == (8192, 8192)
    assert shapes["glu_up_4096x14336"] == (4096, 14336)
    assert shapes["glu_down_14336x4096"] == (14336, 4096)


def test_tiny64_recipe():
    d = WL.generate(WL.by_name("tiny64"))
    assert d["W"].dtype == np.float32 and d["W"].shape == (64, 64)
    assert np.all(d["maxq"] == 15)
    # A and B are sample second moments: symmetric positive semidefinite
    for M in (d["A"], d["B"]):
        assert np.allclose(M, M.T)
        assert np.linalg.eigvalsh(M.astype(np.float64)).min() > -1e-5
    # per-row grid spans the row: min maps to 0, max maps to maxq
    W = d["W"].astype(np.float64)
    lo = W.min(1) / d["scale"] + d["zero"]
    hi = W.max(1) / d["scale"] + d["zero"]
    assert np.allclose(lo, 0, atol=1e-4) and np.allclose(hi, 15, atol=1e-4)


def test_mixed_bits_average():
    spec = WL.by_name("sq8192_mixed")
    # without drawing the full 8192^2 workload: the permutation logic on a
    # reduced copy of the spec with the same ratio of low-bit rows
    small = WL.Spec("mix", 80, 16, "normal", 0.015, 32, True, 3, mixed_low_rows=16)
    d = WL.generate(small)
    assert int((d["maxq"] == 3).sum()) == 16 and int((d["maxq"] == 7).sum()) == 64
    bpw = (spec.mixed_low_rows * 2 + (spec.m - spec.mixed_low_rows) * 3) / spec.m
    assert abs(bpw - 2.80005) < 1e-4
