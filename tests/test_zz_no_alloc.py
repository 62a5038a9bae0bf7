"""bakron_solve_noalloc (through the C ABI) against bakron_solve on the same
inputs: every output agrees bit for bit, on two calls in a row, the second
on a smaller (ragged) layer, so the second call runs on whatever the first
left in the library's scratch.  A problem larger than the fixed scratch is
rejected before anything is enqueued.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (derivation, Theorem 3.2, Corollary 3.4).
"""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B
from oracle import reference as R
from workloads import make_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _problem(m, n, seed):
    d = make_problem(m, n, seed)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    return {"W": to_dev(d["W"]), "LA": to_dev(fa["L"].astype(np.float32)), "PA": to_dev(fa["P"].astype(np.float32)),
            "LB": to_dev(fb["L"].astype(np.float32)), "PB": to_dev(fb["P"].astype(np.float32)),
            "scale": to_dev(d["scale"]), "zero": to_dev(d["zero"]), "maxq": to_dev(d["maxq"])}


def _args(p):
    return (p["W"], p["LA"], p["PA"], p["LB"], p["PB"], p["scale"], p["zero"], p["maxq"])


def test_noalloc_equals_solve_on_two_calls_in_a_row():
    # 1536 x 1024 needs about 72 MiB of the 256 MiB scratch; 200 x 330 is
    # smaller and ragged (padded copies of both factors in the scratch)
    for k, (m, n) in enumerate([(1536, 1024), (200, 330)]):
        p = _problem(m, n, 60 + k)
        print(f"noalloc call {k}: {m}x{n}", flush=True)
        ref = B.solve(*_args(p), want_err=True)
        out = B.solve_noalloc(*_args(p), want_err=True)
        torch.cuda.synchronize()
        for key in ("codes", "V", "err", "objective"):
            assert torch.equal(out[key], ref[key]), ((m, n), key)


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    m, n = 4096, 8192      # 12 m n bytes = 384 MiB > 256 MiB
    assert B.lib().bakron_solve_batch_workspace_bytes is not None
    W = torch.zeros((m, n), device=DEV)
    PA = torch.eye(n, device=DEV)
    PB = torch.eye(m, device=DEV)
    s = torch.ones(m, device=DEV)
    z = torch.zeros(m, device=DEV)
    q = torch.full((m,), 3, dtype=torch.int32, device=DEV)
    with pytest.raises(B.BakronError) as ei:
        B.solve_noalloc(W, None, PA, None, PB, s, z, q, want_objective=False)
    assert ei.value.code == B._binding.BAKRON_ERR_TOO_LARGE
