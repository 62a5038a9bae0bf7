"""The grid contract of the solve calls (include/bakron.h: every scale
finite and > 0, every zero point finite, every maxq in [1, 255]), checked by
the binding on the host before anything is enqueued.  CPU only: the check
takes host tensors or arrays as well as device ones."""
import numpy as np
import pytest
import torch

import two_sided_hessian_amd as B


def _grid(m=6):
    return (torch.full((m,), 0.01), torch.linspace(-2.5, 3.25, m), torch.full((m,), 7, dtype=torch.int32))


def test_valid_grids_pass():
    B.check_grid(*_grid())
    s, z, q = _grid()
    q[0], q[-1] = 1, 255                          # both ends of the code range
    B.check_grid(s, z, q)
    B.check_grid(np.ones(3, np.float32), np.zeros(3, np.float32), np.full(3, 3, np.int32))
    B.check_grid(torch.empty(0), torch.empty(0), torch.empty(0, dtype=torch.int32))   # m = 0


@pytest.mark.parametrize("field,value,what", [
    ("scale", 0.0, "scale must be > 0"),
    ("scale", -0.5, "scale must be > 0"),
    ("scale", float("nan"), "scale must be finite"),
    ("scale", float("inf"), "scale must be finite"),
    ("zero", float("nan"), "zero must be finite"),
    ("zero", float("-inf"), "zero must be finite"),
    ("maxq", 0, "maxq must lie in"),
    ("maxq", -3, "maxq must lie in"),
    ("maxq", 256, "maxq must lie in"),
])
def test_bad_grids_raise(field, value, what):
    s, z, q = _grid()
    {"scale": s, "zero": z, "maxq": q}[field][3] = value
    with pytest.raises(B.GridError, match=what):
        B.check_grid(s, z, q)


def test_grid_error_is_a_value_error():
    assert issubclass(B.GridError, ValueError)
