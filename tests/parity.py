"""Helpers shared by the GPU parity tests (not collected as tests)."""
import numpy as np

import synthetic as S
from oracle import engine as E

# tolerances of the path: relative L2 error per tensor
FWD_TOL = {"fp32": 1e-5, "bf16": 2e-2}
GRAD_TOL = {"fp32": 1e-4, "bf16": 2e-2}


def rel_err(x, ref):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    d = np.linalg.norm((x - ref).ravel())
    n = np.linalg.norm(ref.ravel())
    return d / n if n > 0 else d


def assert_close(x, ref, tol, what=""):
    e = rel_err(x, ref)
    assert e <= tol, f"{what}: rel err {e:.3e} > {tol:.1e} (max abs {np.max(np.abs(np.asarray(x, np.float64) - ref)):.3e})"
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
