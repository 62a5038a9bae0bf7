"""The fused call bakron_quantize (both factorisations and the solve, through
the C ABI) against the three separate calls bakron_factor(A),
bakron_factor(B) and bakron_solve on the same inputs: every output agrees bit
for bit.  The fused call starts the solve on the leading block of each factor
while the factorisations finish on library-owned streams, so the comparison
pins that overlap (and the point where the solve waits for the whole factors)
to the plain order.  Shapes cover dimensions with and without the early
leading block (multiples of 64 above 128, and ragged or small ones), m != n,
degenerate single-row and two-column layers, two calls in a row on one
workspace, factors whose top node runs its last products on the larger
capped grid (a side of 8320: 33 x 33 blocks of 128), and the full 8192^2
workload.

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
SHAPES = [(64, 64), (130, 70), (256, 192), (192, 1024), (1024, 1024), (2048, 640), (1000, 1500), (1, 256),
          (320, 2)]


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def separate(T, want_err=True):
    LA, PA, ia = B.factor(T["A"], 0.01)
    LB, PB, ib = B.factor(T["B"], 0.01)
    out = B.solve(T["W"], LA, PA, LB, PB, T["scale"], T["zero"], T["maxq"], want_err=want_err)
    out.update({"L_A": LA, "P_A": PA, "info_A": ia, "L_B": LB, "P_B": PB, "info_B": ib})
    return out


KEYS = ("codes", "V", "err", "objective", "L_A", "P_A", "info_A", "L_B", "P_B", "info_B")


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{m}x{n}" for m, n in SHAPES])
def test_quantize_equals_separate_calls(shape):
    m, n = shape
    d = make_problem(m, n, 70 + m % 97, global_grid=(n < 4))
    print(f"quantize vs separate: {m}x{n}", flush=True)
    T = {k: to_dev(d[k]) for k in ("W", "A", "B", "scale", "zero", "maxq")}
    ref = separate(T)
    torch.cuda.synchronize()
    ws = B._binding.workspace(B.quantize_workspace_bytes(m, n), torch.device(DEV))
    # two calls in a row on one workspace and stream
    for rep in range(2):
        out = B.quantize(T["W"], T["A"], T["B"], T["scale"], T["zero"], T["maxq"], 0.01, want_err=True, ws=ws)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(out[key], ref[key]), (shape, rep, key)
    assert int(out["info_A"].item()) == 0 and int(out["info_B"].item()) == 0
    # and the result is a valid BaKron rounding (float64 oracle's validator)
    v = R.validate(d["W"], out["codes"].cpu().numpy(), d["scale"], d["zero"], d["maxq"], tau=1e-4,
                   PA=out["P_A"].cpu().numpy().astype(np.float64), PB=out["P_B"].cpu().numpy().astype(np.float64))
    assert v["bad"] == 0 and v["max_step"] <= 1, (shape, v)


def test_quantize_on_a_side_stream():
    # the caller's stream is not the null stream: the library forks its own
    # streams from it and joins them back
    m, n = 512, 768
    d = make_problem(m, n, 5)
    T = {k: to_dev(d[k]) for k in ("W", "A", "B", "scale", "zero", "maxq")}
    ref = separate(T)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = B.quantize(T["W"], T["A"], T["B"], T["scale"], T["zero"], T["maxq"], 0.01, want_err=True,
                         stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(out[key], ref[key]), key


def test_quantize_equals_separate_calls_at_full_size():
    import workloads as WL
    spec = WL.by_name("sq8192_mixed")
    d = WL.generate(spec)
    print(f"quantize vs separate: {spec.name} {spec.m}x{spec.n}", flush=True)
    T = {k: to_dev(d[k]) for k in ("W", "A", "B", "scale", "zero", "maxq")}
    ref = separate(T)
    torch.cuda.synchronize()
    out = B.quantize(T["W"], T["A"], T["B"], T["scale"], T["zero"], T["maxq"], 0.01, want_err=True)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(out[key], ref[key]), key


@pytest.mark.parametrize("shape", [(256, 8320), (8320, 256)], ids=["256x8320", "8320x256"])
def test_quantize_equals_separate_calls_large_top_node(shape):
    # a factor of 8320 has 33 x 33 blocks of 128 at its top node, more than
    # the 1024 the small capped grid takes: its last two products run on the
    # larger capped grid beside the solve
    m, n = shape
    d = make_problem(m, n, 91)
    print(f"quantize vs separate: {m}x{n}", flush=True)
    T = {k: to_dev(d[k]) for k in ("W", "A", "B", "scale", "zero", "maxq")}
    ref = separate(T)
    torch.cuda.synchronize()
    out = B.quantize(T["W"], T["A"], T["B"], T["scale"], T["zero"], T["maxq"], 0.01, want_err=True)
    torch.cuda.synchronize()
    for key in KEYS:
        assert torch.equal(out[key], ref[key]), (shape, key)
    assert int(out["info_A"].item()) == 0 and int(out["info_B"].item()) == 0
