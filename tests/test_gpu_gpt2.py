"""GPT-2-124M shape through the C ABI.

* One sequence of 256 tokens: loss, every logit and all 148 parameter gradients
  against the float64 oracle (fp32 and bf16 variants).
* The timed launch configuration, 8 x 1024 tokens, in both variants: the loss,
  every logit of one sequence and all 148 parameter gradients against the
  oracle's, element by element.  Sequences are independent, so the oracle runs
  them one at a time: the batch loss is the mean of the eight per-sequence mean
  losses (equal lengths), and its gradient the mean of their gradients.  At this
  size the launches are the timed ones: the vocabulary-sized tiles of the LM
  head, its 50,257-row dW, the one-tile-per-CU N = 768 products, the raster
  groups and K splits chosen for 8192 rows.
"""
import gc

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


CHECK_SEQ = 3


@pytest.fixture(scope="module")
def full_oracle():
    """The oracle at 8 x 1024: batch loss, batch gradient of all 148 tensors, and the
    logits of sequence CHECK_SEQ.  The oracle's leaf gradients add up over backward
    passes ([Autograd-1, "Why += and not ="]), so eight passes leave the sum of the
    per-sequence gradients; the batch gradient is that sum / 8.  (About 70 s on 16
    host threads; each pass's graph is collected before the next.)"""
    s, params, ids = S.gpt2(batch=8, seq=1024)
    P = M.as_tensors(params)
    losses, logits_b = [], None
    for b in range(ids.shape[0]):
        loss, logits = M.gpt_loss(P, ids[b:b + 1], s.n_layer, s.n_head)
        loss.backward()
        losses.append(loss.item())
        if b == CHECK_SEQ:
            logits_b = logits.data.reshape(ids.shape[1] - 1, s.vocab).copy()
        del loss, logits
        gc.collect()
    grads = {k: t.grad / ids.shape[0] for k, t in P.items()}
    del P
    gc.collect()
    return s, params, ids, float(np.mean(losses)), logits_b, grads


@pytest.mark.timeout(900)
@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_gpt2_timed_config_against_oracle(big, full_oracle, prec):
    import torch
    s, params, ids, rl, rlog, rgr = full_oracle
    big.set_precision(prec)
    model = G.Gpt(big, s.n_layer, s.n_head, params)
    ids_dev = torch.from_numpy(ids).to("cuda:0")
    inputs, targets = G.split_ids(ids_dev)
    loss, logits = model.loss(inputs, targets)
    big.backward(loss)
    gl = loss.item()
    assert abs(gl - rl) / max(abs(rl), 1) <= FWD_TOL[prec], (gl, rl)
    full = logits.numpy().reshape(ids.shape[0], ids.shape[1] - 1, s.vocab)
    assert_close(full[CHECK_SEQ], rlog, FWD_TOL[prec], f"logits of sequence {CHECK_SEQ}")
    del full
    assert len(model.names) == 148
    worst = 0.0
    for k in model.names:
        worst = max(worst, assert_close(model.P[k].grad(), rgr[k], GRAD_TOL[prec], "grad " + k))
    print(f"{prec} 8x1024: loss {gl:.6f} (oracle {rl:.6f}), worst gradient rel err {worst:.2e}")
    big.tape_reset()
    for t in model.param_list:
        t.release()
    big.set_precision("fp32")
