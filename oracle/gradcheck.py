"""Central-difference gradient check with the pages' error measure.

Test infrastructure only.  Follows [Autograd-1, §"Gradient check"]: clear the
inputs' gradients, run the loss once with backward() for the analytic
gradients, then for every element perturb it by +h and -h (no graph recorded),
take (L+ - L-) / 2h, and compare per input tensor with the norm-wise relative
error ||a - n|| / (||a|| + ||n||); the largest absolute difference is reported
too.  A tensor-valued op is checked through the projection sum(out * R) with a
fixed random R, so that every output element carries its own weight.

The arithmetic runs in the dtype of the inputs: float32 reproduces the pages'
printed numbers, float64 with a small h gives a tight check of the oracle's own
backward rules.
"""
from __future__ import annotations

from typing import Callable, Sequence, Tuple

import numpy as np

from . import engine as E


def run(loss_fn: Callable[[], E.Tensor], inputs: Sequence[E.Tensor], h=1e-2) -> Tuple[float, float]:
    for t in inputs:
        t.zero_grad()
    loss_fn().backward()
    max_abs, max_rel = 0.0, 0.0
    for t in inputs:
        dt = t.data.dtype.type
        hh = dt(h)
        analytic = t.grad_buf().reshape(-1)
        flat = t.data.reshape(-1)
        diff_sq = a_sq = n_sq = 0.0
        for i in range(flat.size):
            old = flat[i]
            with E.no_grad():
                flat[i] = dt(old + hh)
                plus = dt(loss_fn().item())
                flat[i] = dt(old - hh)
                minus = dt(loss_fn().item())
            flat[i] = old
            numeric = dt((plus - minus) / (dt(2) * hh))
            a = dt(analytic[i])
            max_abs = max(max_abs, float(abs(a - numeric)))
            d = float(a) - float(numeric)
            diff_sq += d * d
            a_sq += float(a) * float(a)
            n_sq += float(numeric) * float(numeric)
        denom = np.sqrt(a_sq) + np.sqrt(n_sq)
        if denom > 0:
            max_rel = max(max_rel, float(np.sqrt(diff_sq) / denom))
    return max_abs, max_rel


def forward_difference(f, x, h):
    """(f(x + h) - f(x)) / h in the arithmetic of x and h."""
    return (f(x + h) - f(x)) / h


def central_difference(f, x, h):
    """(f(x + h) - f(x - h)) / 2h in the arithmetic of x and h; the derivative
    estimate the check uses ([Autograd-1, §"The derivative"])."""
    return (f(x + h) - f(x - h)) / (type(h)(2) * h)


def projected(op_out: Callable[[], E.Tensor], R: np.ndarray) -> Callable[[], E.Tensor]:
    """Loss sum(op(...) * R) for checking an op with a tensor output."""
    Rt = E.Tensor(R)
    return lambda: E.sum_all(E.mul(op_out(), Rt))
