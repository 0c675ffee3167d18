"""GPT-2-124M shape through the C ABI.

* One sequence of 256 tokens: loss, every logit and all 148 parameter gradients
  against the float64 oracle (fp32 and bf16 variants).
* The timed launch configuration (8 x 1024 tokens): sampled logit rows of one
  sequence against the oracle's forward of that sequence (sequences are
  independent in the forward), and the gradient checked at full size by a
  central finite difference of the GPU's own loss along the computed gradient.
  The bf16 variant's 148 gradients at that size are checked against the fp32
  variant's (the kernels and tilings this size selects differ from the
  256-token case's).
"""
import numpy as np
import pytest

import synthetic as S
from oracle import engine as E
from oracle import models as M
from parity import FWD_TOL, GRAD_TOL, assert_close

pytestmark = pytest.mark.gpu

T = pytest.importorskip("transformer_fwd_bwd_amd")
from transformer_fwd_bwd_amd import gpt as G  # noqa: E402


@pytest.fixture(scope="module")
def big():
    from conftest import gpu_available
    if not gpu_available():
        pytest.skip("no GPU")
    c = T.Context(arena_bytes=48 << 30, precision="fp32")
    yield c
    c.close()


@pytest.fixture(scope="module")
def short_oracle():
    s, params, ids = S.gpt2(batch=1, seq=256)
    P = M.as_tensors(params)
    loss, logits = M.gpt_loss(P, ids, s.n_layer, s.n_head)
    loss.backward()
    return s, params, ids, loss.item(), logits.data, {k: t.grad for k, t in P.items()}


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_gpt2_shape_step_parity(big, short_oracle, prec):
    s, params, ids, rl, rlog, rgr = short_oracle
    big.set_precision(prec)
    model = G.Gpt(big, s.n_layer, s.n_head, params)
    inputs, targets = G.split_ids(ids)
    loss, logits = model.loss(inputs, targets)
    big.backward(loss)
    tol_f, tol_g = FWD_TOL[prec], GRAD_TOL[prec]
    assert abs(loss.item() - rl) / max(abs(rl), 1) <= tol_f
    assert_close(logits.numpy(), rlog.reshape(logits.shape), tol_f, "logits")
    worst = 0.0
    for k in model.names:
        worst = max(worst, assert_close(model.P[k].grad(), rgr[k], tol_g, "grad " + k))
    print(f"{prec}: worst gradient rel err {worst:.2e}")
    big.tape_reset()
    for t in model.param_list:
        t.release()
    big.set_precision("fp32")


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_gpt2_full_launch_config(big, prec):
    s, params, ids = S.gpt2(batch=8, seq=1024)
    big.set_precision(prec)
    model = G.Gpt(big, s.n_layer, s.n_head, params)
    import torch
    ids_dev = torch.from_numpy(ids).to("cuda:0")
    inputs, targets = G.split_ids(ids_dev)
    loss, logits = model.loss(inputs, targets)
    big.backward(loss)
    gl = loss.item()
    assert np.isfinite(gl) and abs(gl - np.log(s.vocab)) < 0.5

    # sampled rows of sequence 3 against the oracle's forward of that sequence alone
    b, rows = 3, [0, 1, 511, 1023]
    full = logits.numpy().reshape(8, 1024, s.vocab)
    with E.no_grad():
        ref = M.gpt_logits(M.as_tensors(params), ids[b:b + 1, :-1], s.n_layer, s.n_head).data[0]
    assert_close(full[b, rows], ref[rows], FWD_TOL[prec], "logit rows")

    if prec == "fp32":
        # directional derivative of the full-batch loss along the computed gradient itself:
        # (L(p + e v) - L(p - e v)) / 2e must equal <grad, v> = |grad| for v = grad/|grad|;
        # e is chosen so that the loss moves by about 1e-3 (well above fp32 rounding of the loss)
        names = ["h.11.mlp.c_proj.bias", "ln_f.weight", "h.0.attn.c_attn.weight", "wte.weight"]
        grads = {k: model.P[k].grad() for k in names}
        big.tape_reset()
        big.set_grad_enabled(False)
        for k in names:
            p0 = params[k]
            gn = float(np.linalg.norm(grads[k].astype(np.float64)))
            assert gn > 0
            v = (grads[k] / gn).astype(np.float32)
            eps = 1e-3 / gn
            vals = []
            for sgn in (1, -1):
                model.P[k].write(p0 + sgn * eps * v)
                vals.append(model.loss(inputs, targets)[0].item())
                big.tape_reset()
            model.P[k].write(p0)
            fd = (vals[0] - vals[1]) / (2 * eps)
            an = float(np.sum(grads[k].astype(np.float64) * v))
            assert abs(fd - an) <= 2e-2 * abs(an), (k, fd, an)
        big.set_grad_enabled(True)
    big.tape_reset()
    for t in model.param_list:
        t.release()
    big.set_precision("fp32")


def test_gpt2_full_launch_config_bf16_gradients(big):
    """All 148 parameter gradients of the bf16 variant at 8 x 1024 tokens (the tile
    shapes, raster groups, bf16-only intermediates and deferred column sums of the
    timed configuration) against the fp32 variant's on the same batch, within the
    bf16 tolerance; the fp32 gradient is itself checked above by finite differences."""
    s, params, ids = S.gpt2(batch=8, seq=1024)
    import torch
    ids_dev = torch.from_numpy(ids).to("cuda:0")
    inputs, targets = G.split_ids(ids_dev)
    grads = {}
    for prec in ("fp32", "bf16"):
        big.set_precision(prec)
        model = G.Gpt(big, s.n_layer, s.n_head, params)
        loss, _ = model.loss(inputs, targets)
        big.backward(loss)
        grads[prec] = {k: model.P[k].grad() for k in model.names}
        big.tape_reset()
        for t in model.param_list:
            t.release()
    big.set_precision("fp32")
    assert len(grads["bf16"]) == 148
    for k, g32 in grads["fp32"].items():
        assert_close(grads["bf16"][k], g32, GRAD_TOL["bf16"], k)
