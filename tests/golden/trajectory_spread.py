"""Spread between two valid BaKron trajectories of the same layer.

Runs the float64 oracle twice per workload: with the float64 factors P_A,
P_B, and with the same factors rounded to float32 (a relative change of at
most 2^-24 per entry, the precision the GPU factors are stored in).  Both
runs are exact BaKron computations; where they differ, the difference is
the sensitivity of the rounding trajectory itself: one decision that lands
on the other side of a boundary changes the error fed to every entry below
and to the right of it (paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians", derivation of the bottom-right update), and
those changes can flip further decisions.

Writes trajectory_spread.json next to this file: per workload, the fraction
of differing codes, the largest code difference and the relative difference
of the objective ||L_B (V - W) L_A^T||_F^2.  Calls only oracle/ and
workloads/.  Usage: python tests/golden/trajectory_spread.py
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


def spread(name):
    d = WL.generate(WL.by_name(name))
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    args = (d["scale"], d["zero"], d["maxq"])
    c64, V64, _ = O2.bakron_recursive(d["W"], fa["P"], fb["P"], *args)
    PA32 = fa["P"].astype(np.float32).astype(np.float64)
    PB32 = fb["P"].astype(np.float32).astype(np.float64)
    c32, V32, _ = O2.bakron_recursive(d["W"], PA32, PB32, *args)
    o64 = R.objective(d["W"], V64, fa["L"], fb["L"])
    o32 = R.objective(d["W"], V32, fa["L"], fb["L"])
    return {"differ_frac": float(np.mean(c64 != c32)), "max_step": int(np.abs(c64 - c32).max()),
            "objective_rel": float(abs(o64 - o32) / o64)}


if __name__ == "__main__":
    O2.build()
    res = {}
    for name in NAMES:
        res[name] = spread(name)
        print(name, res[name], flush=True)
    with open(os.path.join(HERE, "trajectory_spread.json"), "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
