"""Spread between valid BaKron trajectories of the same layer.

Runs the float64 oracle on each workload with three versions of the factors
P_A, P_B and compares the results:
* the float64 factors;
* the same factors rounded to float32 (a relative change of at most 2^-24
  per entry): keys differ_frac, max_step, objective_rel;
* factors computed in float32 arithmetic by LAPACK (oracle.reference.
  factor_float32, independent of the GPU path), whose errors, about
  n u cond(A_d), are of the kind any float32 solver's factors carry: keys
  lapack32_differ_frac, lapack32_max_step, lapack32_objective_rel.
Every run is an exact BaKron computation on its factors; where they differ,
the difference is the sensitivity of the rounding trajectory itself: one
decision that lands on the other side of a boundary changes the error fed to
every entry below and to the right of it (paper summary "FastKron: Efficient
Quantization with Kronecker-Factored Hessians", derivation of the
bottom-right update; Theorem 3.2's equality holds in exact arithmetic), and
those changes can flip further decisions.

Writes trajectory_spread.json next to this file (after each workload):
per workload, the fraction of differing codes, the largest code difference
and the relative difference of the objective ||L_B (V - W) L_A^T||_F^2
(measured with the float64 factors' L).  Calls only oracle/ and workloads/.
Usage: python tests/golden/trajectory_spread.py [--only-lapack32] [names...]
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import workloads as WL  # noqa: E402
from oracle import recursive as O2  # noqa: E402
from oracle import reference as R  # noqa: E402

NAMES = ("tiny64", "sq1024", "sq4096_t5", "glu_up_4096x14336", "glu_down_14336x4096", "sq8192_mixed")
OUT = os.path.join(HERE, "trajectory_spread.json")


def _compare(d, fa, fb, c64, V64, c, V):
    o64 = R.objective(d["W"], V64, fa["L"], fb["L"])
    o = R.objective(d["W"], V, fa["L"], fb["L"])
    return float(np.mean(c64 != c)), int(np.abs(c64 - c).max()), float(abs(o64 - o) / o64)


def spread(name, only_lapack32=False):
    d = WL.generate(WL.by_name(name))
    args = (d["scale"], d["zero"], d["maxq"])
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    c64, V64, _ = O2.bakron_recursive(d["W"], fa["P"], fb["P"], *args)
    res = {}
    if not only_lapack32:
        PA32 = fa["P"].astype(np.float32).astype(np.float64)
        PB32 = fb["P"].astype(np.float32).astype(np.float64)
        c32, V32, _ = O2.bakron_recursive(d["W"], PA32, PB32, *args)
        res["differ_frac"], res["max_step"], res["objective_rel"] = _compare(d, fa, fb, c64, V64, c32, V32)
    ga, gb = R.factor_float32(d["A"]), R.factor_float32(d["B"])
    cl, Vl, _ = O2.bakron_recursive(d["W"], ga["P"].astype(np.float64), gb["P"].astype(np.float64), *args)
    (res["lapack32_differ_frac"], res["lapack32_max_step"],
     res["lapack32_objective_rel"]) = _compare(d, fa, fb, c64, V64, cl, Vl)
    return res


if __name__ == "__main__":
    O2.build(force=False)
    only = "--only-lapack32" in sys.argv
    names = [a for a in sys.argv[1:] if not a.startswith("--")] or list(NAMES)
    res = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for name in names:
        res.setdefault(name, {}).update(spread(name, only))
        print(name, res[name], flush=True)
        with open(OUT, "w") as f:
            json.dump(res, f, indent=1)
            f.write("\n")
