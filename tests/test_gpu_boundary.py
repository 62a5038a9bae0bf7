"""The boundary's stream and grid contracts, on the GPU through the C ABI.

* bakron_solve on many fresh caller streams: the library's own streams are a
  fixed pool per device, and every call gives the single-stream result bit
  for bit;
* bakron_solve_batch on fresh streams with no manual joins by the caller:
  the binding orders the batch streams after the current stream and joins
  them back, so the outputs equal bakron_solve's bit for bit once the current
  stream is synchronised;
* a grid outside the contract raises before anything is enqueued.

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


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _problem(m, n, seed):
    d = make_problem(m, n, seed)
    fa, fb = R.factor(d["A"]), R.factor(d["B"])
    return {"W": to_dev(d["W"]), "LA": to_dev(fa["L"].astype(np.float32)), "PA": to_dev(fa["P"].astype(np.float32)),
            "LB": to_dev(fb["L"].astype(np.float32)), "PB": to_dev(fb["P"].astype(np.float32)),
            "scale": to_dev(d["scale"]), "zero": to_dev(d["zero"]), "maxq": to_dev(d["maxq"])}


def _solve(p, **kw):
    return B.solve(p["W"], p["LA"], p["PA"], p["LB"], p["PB"], p["scale"], p["zero"], p["maxq"], want_err=True, **kw)


def test_solve_on_many_fresh_streams():
    # 1536 x 1024: 39 tile anti-diagonals, so the upper nodes are split and
    # their far parts use the library's streams
    p = _problem(1536, 1024, 81)
    ref = _solve(p)
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()
    for k in range(100):
        s = torch.cuda.Stream()
        s.wait_stream(main)
        with torch.cuda.stream(s):
            out = _solve(p, stream=s, check=False)
        main.wait_stream(s)
        if k % 25 == 0 or k == 99:
            torch.cuda.synchronize()
            for key in ("codes", "V", "err", "objective"):
                assert torch.equal(out[key], ref[key]), (k, key)
    print("100 solves on fresh streams equal the single-stream result", flush=True)


def test_batch_on_fresh_streams_needs_no_joins():
    shapes = [(256, 192), (1024, 1024), (130, 70), (512, 640)]
    probs = [_problem(m, n, 90 + k) for k, (m, n) in enumerate(shapes)]
    refs = [_solve(p) for p in probs]
    torch.cuda.synchronize()
    for rep in range(3):
        streams = [torch.cuda.Stream() for _ in range(3)]
        # the inputs are rewritten on the current stream right before the call
        for p in probs:
            p["W"].mul_(1.0)
        outs = B.solve_batch(probs, streams, want_err=True)
        torch.cuda.current_stream().synchronize()   # only the current stream
        for k in range(len(probs)):
            for key in ("codes", "V", "err", "objective"):
                assert torch.equal(outs[k][key], refs[k][key]), (rep, shapes[k], key)


@pytest.mark.parametrize("field,value", [("scale", 0.0), ("scale", float("nan")), ("zero", float("inf")),
                                         ("maxq", 256), ("maxq", 0)])
def test_bad_grid_raises_before_enqueue(field, value):
    p = _problem(64, 128, 3)
    p[field][5] = value
    with pytest.raises(B.GridError):
        _solve(p)
    with pytest.raises(B.GridError):
        B.gptq(p["W"], p["LA"], p["PA"], p["scale"], p["zero"], p["maxq"])
    with pytest.raises(B.GridError):
        B.solve_batch([p])
