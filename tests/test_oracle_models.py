"""Pins of the oracle's compositions: model shapes, whole-model finite
differences, the KV-cache invariant, AdamW closed forms and the sampler.  CPU only."""
import math

import numpy as np
import pytest

import synthetic as S
from oracle import decode as D
from oracle import engine as E
from oracle import gradcheck as G
from oracle import models as M
from oracle import optim as OPT
from oracle import ops as O


def test_gpt2_shape_pins(golden):
    fx = golden("gpt2_shapes.json")
    shapes = S.gpt_param_shapes(S.GPT2_124M)
    assert len(shapes) == fx["n_tensors"]
    assert M.param_count(shapes) == fx["n_params"]
    d = dict(shapes)
    for k, v in fx["shapes"].items():
        assert list(d[k]) == v
    # block multiply-adds per token, from the weight shapes: about 85 million
    macs = sum(int(np.prod(s)) for n, s in shapes if n.startswith("h.") and n.endswith("weight") and len(s) == 2)
    assert macs == 84934656
    assert abs(macs - fx["block_macs_per_token_approx"]) / fx["block_macs_per_token_approx"] < 0.01


def test_workload_param_counts():
    p, _, _ = S.tiny_mlp()
    assert sum(a.size for a in p.values()) == 1732
    assert sum(a.size for a in S.char_mlp().values()) == 67392
    assert M.param_count(S.gpt_param_shapes(S.TINY_GPT)) == 413184


def _mini_gpt(seed=5, std=0.3):
    s = S.GptShape(vocab=11, n_positions=6, n_layer=2, n_head=2, n_embd=8)
    params = S.gpt_params(s, seed, std=std)
    rng = S.rng_for(seed + 1)
    for k, v in params.items():            # non-trivial LN gains and biases for the check
        if v.ndim == 1:
            params[k] = (v + 0.2 * rng.standard_normal(v.shape)).astype(np.float32)
    ids = S.token_batch(seed + 2, 2, 5, s.vocab)
    return s, params, ids


def test_whole_gpt_gradients_match_central_differences():
    s, params, ids = _mini_gpt()
    P = M.as_tensors(params)
    loss_fn = lambda: M.gpt_loss(P, ids, s.n_layer, s.n_head)[0]
    for t in P.values():
        t.zero_grad()
    loss_fn().backward()
    rng = S.rng_for(77)
    worst = 0.0
    for name, t in P.items():
        assert t.grad is not None, name          # every parameter reaches the loss
        flat = t.data.reshape(-1)
        for i in rng.choice(flat.size, size=min(4, flat.size), replace=False):
            old = flat[i]
            with E.no_grad():
                flat[i] = old + 1e-5
                lp = loss_fn().item()
                flat[i] = old - 1e-5
                lm = loss_fn().item()
            flat[i] = old
            num = (lp - lm) / 2e-5
            a = t.grad.reshape(-1)[i]
            worst = max(worst, abs(a - num) / max(abs(a) + abs(num), 1e-8))
    assert worst < 1e-6


def test_tiny_mlp_and_char_mlp_gradients_fd():
    p, x, y = S.tiny_mlp()
    P = M.as_tensors(p)
    _, rel = G.run(lambda: M.tiny_mlp_loss(P, x, y)[0], list(P.values()), h=1e-5)
    assert rel < 1e-8
    cp = M.as_tensors(S.char_mlp())
    ctx, tgt = S.char_mlp_batch(0, batch=6)
    small = {k: v for k, v in cp.items()}
    _, rel = G.run(lambda: M.char_mlp_loss(small, ctx, tgt)[0], [small["emb"], small["b1"], small["b2"]], h=1e-5)
    assert rel < 1e-8


def test_kv_cache_step_equals_full_forward():
    """[GPT2-4, §"Generation with KV cache"]: the cached path is the same
    computation as the full forward, position by position."""
    s, params, ids = _mini_gpt(std=0.5)
    P64 = {k: v.astype(np.float64) for k, v in params.items()}
    inp = ids[:, :5]
    with E.no_grad():
        full = M.gpt_logits(M.as_tensors(params), inp, s.n_layer, s.n_head).data
    cache = D.KvCache(s.n_layer)
    for pos in range(5):
        step_logits = D.step(P64, inp[:, pos], pos, cache, s.n_layer, s.n_head)
        assert np.allclose(step_logits, full[:, pos], rtol=1e-12, atol=1e-12)


def test_uniform_logits_loss_is_log_vocab_on_model():
    s, params, ids = _mini_gpt()
    for k in params:
        if k.endswith("weight") and params[k].ndim == 2 and k != "wte.weight":
            params[k][...] = 0
    params["ln_f.weight"][...] = 0
    params["ln_f.bias"][...] = 0
    loss, _ = M.gpt_loss(M.as_tensors(params), ids, s.n_layer, s.n_head)
    assert abs(loss.item() - math.log(s.vocab)) < 1e-12


# --------------------------------------------------------------------------
# Optimizers
# --------------------------------------------------------------------------
def test_adamw_constant_gradient_closed_form():
    """For a constant gradient g, m/bc1 = g and v/bc2 = g^2 at every step, so each
    step moves p by -lr (g / (|g| + eps) + wd p)."""
    rng = S.rng_for(3)
    w = E.Tensor(rng.standard_normal((4, 3)))
    b = E.Tensor(rng.standard_normal((3,)))
    g_w, g_b = rng.standard_normal((4, 3)), rng.standard_normal((3,))
    opt = OPT.AdamW([w, b], lr=1e-3, weight_decay=0.01)
    pw, pb = w.data.copy(), b.data.copy()
    for _ in range(5):
        w.grad, b.grad = g_w.copy(), g_b.copy()
        opt.step()
        pw = pw - 1e-3 * (g_w / (np.abs(g_w) + 1e-8) + 0.01 * pw)
        pb = pb - 1e-3 * (g_b / (np.abs(g_b) + 1e-8))
        assert np.allclose(w.data, pw, rtol=1e-10, atol=1e-13)
        assert np.allclose(b.data, pb, rtol=1e-10, atol=1e-13)


def test_adamw_zero_gradient_and_missing_gradient():
    w = E.Tensor(np.full((2, 2), 3.0))
    b = E.Tensor(np.full((2,), 3.0))
    c = E.Tensor(np.full((2, 2), 3.0))       # never gets a gradient: skipped
    opt = OPT.AdamW([w, b, c], lr=0.1, weight_decay=0.5)
    w.grad, b.grad = np.zeros((2, 2)), np.zeros(2)
    opt.step()
    assert np.allclose(w.data, 3.0 * (1 - 0.1 * 0.5))
    assert np.array_equal(b.data, np.full(2, 3.0))
    assert np.array_equal(c.data, np.full((2, 2), 3.0))


def test_sgd_step():
    w = E.Tensor(np.array([1.0, 2.0]))
    w.grad = np.array([0.5, -1.0])
    OPT.SGD([w], lr=0.1).step()
    assert np.allclose(w.data, [0.95, 2.1])


def test_adamw_trains_circle_classifier():
    """[Autograd-1, §"Training loop"]: the 2->16->2 network with AdamW (lr 0.05,
    no weight decay) separates the circle x^2 + y^2 < 0.5; the pages' random
    streams cannot be reproduced, so only the qualitative outcome is pinned
    (loss well under the SGD run's, accuracy near 100%)."""
    rng = S.rng_for(11)
    xs = rng.uniform(-1, 1, size=(256, 2))
    ys = ((xs ** 2).sum(1) < 0.5).astype(np.int64)

    def train(adam):
        r = S.rng_for(12)
        P = [E.Tensor(r.standard_normal((2, 16)) * 0.5), E.Tensor(np.zeros(16)),
             E.Tensor(r.standard_normal((16, 2)) * 0.5), E.Tensor(np.zeros(2))]
        opt = OPT.AdamW(P, lr=0.05, weight_decay=0.0) if adam else OPT.SGD(P, lr=0.05)
        X = E.Tensor(xs)
        for _ in range(501):
            h = E.tanh(E.add(E.matmul(X, P[0]), P[1]))
            logits = E.add(E.matmul(h, P[2]), P[3])
            loss = E.softmax_cross_entropy(logits, ys)
            opt.zero_grad()
            loss.backward()
            opt.step()
        return loss.item(), (logits.data.argmax(1) == ys).mean()
    l_sgd, _ = train(False)
    l_adam, acc = train(True)
    assert l_adam < 0.1 and acc > 0.97 and l_adam < l_sgd


# --------------------------------------------------------------------------
# Sampling
# --------------------------------------------------------------------------
def test_top_k_keeps_ties_and_masks_the_rest():
    l = np.array([1.0, 5.0, 3.0, 5.0, 3.0, -2.0])
    p = D.top_k_temperature_probs(l, 2, 1.0)
    assert np.count_nonzero(p) == 2 and p[1] == p[3] == 0.5
    p3 = D.top_k_temperature_probs(l, 3, 1.0)
    assert np.count_nonzero(p3) == 4          # the tie at the 3rd value survives
    assert abs(p3.sum() - 1) < 1e-15


def test_top_k_1_is_argmax_and_k0_is_plain_softmax():
    l = S.random_array(5, (50,), 2.0, dtype=np.float64)
    for u in (0.0, 0.3, 0.999999):
        assert D.sample(D.top_k_temperature_probs(l, 1, 1.0), u) == int(np.argmax(l))
    p = D.top_k_temperature_probs(l, 0, 1.0)
    e = np.exp(l - l.max())
    assert np.allclose(p, e / e.sum(), atol=1e-16)
    # temperature divides the (masked) logits
    p2 = D.top_k_temperature_probs(l, 0, 2.0)
    e2 = np.exp((l - l.max()) / 2)
    assert np.allclose(p2, e2 / e2.sum(), atol=1e-16)


def test_inverse_cdf_measure_equals_probability():
    p = D.top_k_temperature_probs(S.random_array(6, (12,), dtype=np.float64), 5, 0.8)
    us = (np.arange(200000) + 0.5) / 200000
    counts = np.bincount([D.sample(p, u) for u in us], minlength=12) / us.size
    assert np.allclose(counts, p, atol=2e-5)
