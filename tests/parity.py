"""Helpers shared by the GPU parity tests (not collected as tests).

Every comparison of a GPU result x with the oracle's r passes two gates:

* relative L2 error per tensor, ||x - r||_2 / ||r||_2 <= tol, with tol the
  path's stated tolerance: 1e-5 for fp32 forward values, 1e-4 for fp32
  gradients and updated parameters, 2e-2 for the bf16-MFMA variant;
* an element-wise bound, |x_i - r_i| <= tol * (|r_i| + ELEM_A * s_i) for
  every element, where s_i is the larger of the RMS of the row (last axis)
  that element i sits in and the RMS of the whole tensor.  The absolute part
  is there because a sum's rounding error scales with the magnitude of the
  terms summed, not with the (possibly tiny) element it lands on: an element
  near zero carries about as much absolute error as its neighbours.  The
  tensor's RMS is the floor because the activations every row is built from
  carry errors at their own scale (a row of a weight gradient whose input
  feature is small still inherits that absolute error); the row's RMS takes
  over where a row is much larger than the rest (the rows of the tied
  embedding's gradient for the tokens in the batch are ~15x the tensor's RMS,
  and their rounding errors scale with them).  Eight such units leave room
  for the tail of the error over hundreds of millions of elements while still
  catching one wrong row, column or ragged tile, whose elements err by about
  one unit each (a gate of 2e-2 * 9 = 0.18 units in bf16, 9e-4 in fp32
  gradients).

Each check's achieved errors, as fractions of its tolerance, are recorded in
RESULTS; the test session prints them at its end (tests/conftest.py).
"""
import os

import numpy as np

from oracle import engine as E

# tolerances of the path: relative L2 error per tensor
FWD_TOL = {"fp32": 1e-5, "bf16": 2e-2}
GRAD_TOL = {"fp32": 1e-4, "bf16": 2e-2}
ELEM_A = 8.0

# (test id, what, L2 error / tol, element-wise error / tol)
RESULTS = []


def bf16_round(a):
    """float32 -> nearest-even bf16 -> float32, in numpy (the rounding the kernels apply)."""
    b = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return (b << 16).astype(np.uint32).view(np.float32)


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    d = np.linalg.norm((x - ref).ravel())
    n = np.linalg.norm(ref.ravel())
    if n == 0:
        return 0.0 if d == 0 else float("inf")   # an all-zero reference must be matched exactly
    return d / n


def elem_err(x, ref):
    """max_i |x_i - r_i| / (|r_i| + ELEM_A * s_i), s_i = max(RMS of element i's row, RMS of the
    tensor): the smallest tol the element-wise gate passes at."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rows = ref.reshape(-1, ref.shape[-1]) if ref.ndim >= 2 else ref.reshape(1, -1)
    xr = x.reshape(rows.shape)
    rms = float(np.sqrt(np.mean(rows * rows)))
    num = np.abs(xr - rows)
    if rms == 0.0:
        return 0.0 if num.max() == 0 else float("inf")
    s = np.maximum(np.sqrt(np.mean(rows * rows, axis=1, keepdims=True)), rms)
    return float(np.max(num / (np.abs(rows) + ELEM_A * s)))


def assert_close(x, ref, tol, what=""):
    x = np.asarray(x)
    ref = np.asarray(ref)
    assert x.shape == ref.shape, (what, x.shape, ref.shape)
    e = rel_err(x, ref)
    el = elem_err(x, ref)
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    RESULTS.append((test, what, e / tol, el / tol))
    assert np.all(np.isfinite(np.asarray(x, np.float64))), f"{what}: non-finite values"
    assert e <= tol, f"{what}: rel L2 err {e:.3e} > {tol:.1e} (max abs {np.max(np.abs(np.asarray(x, np.float64) - ref)):.3e})"
    if el > tol:
        xv = np.asarray(x, np.float64).reshape(-1)
        rv = np.asarray(ref, np.float64).reshape(-1)
        i = int(np.argmax(np.abs(xv - rv)))
        raise AssertionError(f"{what}: element-wise err {el:.3e} > {tol:.1e} (|x-r| <= tol*(|r| + {ELEM_A:g}*s)); "
                             f"largest |x-r| at flat index {i}: x {xv[i]:.6e} r {rv[i]:.6e}")
    return e


def gpu_op_with_grads(ctx, build, arrays, R):
    """Run build(*tensors) on the GPU, take loss = sum(out * R), backward; return out and input grads."""
    import transformer_fwd_bwd_amd as T
    ts = [ctx.tensor(a.shape, a) for a in arrays]
    out = build(*ts)
    Rt = ctx.tensor(R.shape, R)
    loss = T.sum_all(T.mul(out, Rt))
    ctx.backward(loss)
    res = out.numpy(), [t.grad() for t in ts]
    ctx.tape_reset()
    for t in ts + [Rt]:
        t.release()
    return res


def oracle_op_with_grads(build, arrays, R):
    ts = [E.Tensor(np.asarray(a, np.float64)) for a in arrays]
    out = build(*ts)
    loss = E.sum_all(E.mul(out, E.Tensor(np.asarray(R, np.float64))))
    loss.backward()
    return out.data, [t.grad for t in ts]
