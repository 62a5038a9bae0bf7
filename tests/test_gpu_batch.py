"""Batched solves of independent layers (bakron_solve_batch, through the C
ABI): every layer's outputs equal bakron_solve's on the same inputs, bit for
bit, whatever the stream a layer lands on, and pass the float64 oracle's
validator.  A batch layer runs all its work on its own stream, while
bakron_solve runs the far parts of its upper recursion nodes on separate
streams (shapes with at least 16 tile anti-diagonals), so the comparison
also pins the split schedule to the unsplit one, padded shapes included.

Pages: [S] paper summary "FastKron: Efficient Quantization with
Kronecker-Factored Hessians" (every linear layer has its own W, A and B).
"""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B
from oracle import reference as R
from workloads import make_problem

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SHAPES = [(64, 64), (130, 70), (256, 192), (1024, 1024), (96, 300), (1, 64), (512, 512), (1000, 1500),
          (2048, 640)]


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("n_streams", [1, 3])
def test_batch_equals_single_solves(n_streams):
    probs, hosts = [], []
    for k, (m, n) in enumerate(SHAPES):
        d = make_problem(m, n, 40 + k, global_grid=(n == 1))
        fa, fb = R.factor(d["A"]), R.factor(d["B"])
        hosts.append((d, fa["P"].astype(np.float32), fb["P"].astype(np.float32)))
        probs.append({"W": to_dev(d["W"]), "LA": to_dev(fa["L"].astype(np.float32)),
                      "PA": to_dev(fa["P"].astype(np.float32)), "LB": to_dev(fb["L"].astype(np.float32)),
                      "PB": to_dev(fb["P"].astype(np.float32)), "scale": to_dev(d["scale"]),
                      "zero": to_dev(d["zero"]), "maxq": to_dev(d["maxq"])})
    streams = [torch.cuda.Stream() for _ in range(n_streams)]
    main = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(main)
    outs = B.solve_batch(probs, streams, want_err=True)
    for s in streams:
        main.wait_stream(s)
    torch.cuda.synchronize()
    for k, p in enumerate(probs):
        ref = B.solve(p["W"], p["LA"], p["PA"], p["LB"], p["PB"], p["scale"], p["zero"], p["maxq"], want_err=True)
        torch.cuda.synchronize()
        for key in ("codes", "V", "err", "objective"):
            assert torch.equal(outs[k][key], ref[key]), (SHAPES[k], key)
        d, PA, PB = hosts[k]
        v = R.validate(d["W"], outs[k]["codes"].cpu().numpy(), d["scale"], d["zero"], d["maxq"], tau=1e-4,
                       PA=PA.astype(np.float64), PB=PB.astype(np.float64))
        assert v["bad"] == 0 and v["max_step"] <= 1, (SHAPES[k], v)


@pytest.mark.parametrize("name", ["sq4096_t5", "sq8192_mixed"])
def test_split_schedule_equals_unsplit_at_full_size(name):
    # bakron_solve cuts the upper nodes' propagation into parts run on
    # library-owned streams; a batch layer runs the same kernels unsplit on
    # its stream.  At the full workload sizes every output must agree bit for
    # bit (the parts sum the same products in the same order).
    import workloads as WL
    spec = WL.by_name(name)
    d = WL.generate(spec)
    print(f"split vs unsplit: {name} {spec.m}x{spec.n}", flush=True)
    A, Bm = to_dev(d["A"]), to_dev(d["B"])
    LA, PA, ia = B.factor(A, 0.01)
    LB, PB, ib = B.factor(Bm, 0.01)
    torch.cuda.synchronize()
    assert int(ia.item()) == 0 and int(ib.item()) == 0
    prob = {"W": to_dev(d["W"]), "LA": LA, "PA": PA, "LB": LB, "PB": PB, "scale": to_dev(d["scale"]),
            "zero": to_dev(d["zero"]), "maxq": to_dev(d["maxq"])}
    ref = B.solve(prob["W"], LA, PA, LB, PB, prob["scale"], prob["zero"], prob["maxq"], want_err=True)
    torch.cuda.synchronize()
    (out,) = B.solve_batch([prob], [torch.cuda.current_stream()], want_err=True)
    torch.cuda.synchronize()
    for key in ("codes", "V", "err", "objective"):
        assert torch.equal(out[key], ref[key]), key
