"""bakron_solve_noalloc under HIP graph capture (through the C ABI): it
allocates nothing and enqueues only kernels on the caller's stream, so the
whole solve can be captured once and replayed.  Every replay, with eager work
on the outputs between replays, equals the eager call bit for bit.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (derivation, Theorem 3.2).
"""
import time

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


@pytest.mark.parametrize("m,n", [(1024, 1024), (200, 330)])
def test_noalloc_solve_replays_from_a_graph(m, n):
    d = make_problem(m, n, 700 + m)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    args = [to_dev(x) for x in (d["W"], fa["L"].astype(np.float32), fa["P"].astype(np.float32),
                                fb["L"].astype(np.float32), fb["P"].astype(np.float32), d["scale"], d["zero"],
                                d["maxq"])]
    B.check_grid(*args[5:])
    out = {"V": torch.empty((m, n), device=DEV), "codes": torch.empty((m, n), dtype=torch.uint8, device=DEV),
           "err": torch.empty((m, n), device=DEV), "objective": torch.empty(1, dtype=torch.float64, device=DEV)}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # eager call (looks the scratch up) on the stream the capture will use
        B.solve_noalloc(*args, out=out, want_err=True, check=False)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        B.solve_noalloc(*args, out=out, want_err=True, check=False)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in out.values():
            v.zero_()                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], ref[k]), (rep, k)
    # eager calls against replays (informational)
    reps = 10
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        B.solve_noalloc(*args, out=out, want_err=True, check=False)
    torch.cuda.synchronize()
    t_eager = (time.perf_counter() - t0) / reps
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    t_graph = (time.perf_counter() - t0) / reps
    print(f"{m}x{n}: eager {t_eager * 1e3:.3f} ms per solve, graph replay {t_graph * 1e3:.3f} ms", flush=True)
    for k in out:
        assert torch.equal(out[k], ref[k]), k
