"""Workload parity: tiny MLP, char-level MLP LM and tiny GPT through the C ABI
against the float64 oracle -- forward, loss, every gradient, and the AdamW
update (teacher-forced per step: both sides start each step from the GPU's
parameters)."""
import numpy as np
import pytest

import synthetic as S
from oracle import engine as E
from oracle import models as M
from oracle import optim as OPT
from parity import FWD_TOL, GRAD_TOL, assert_close

pytestmark = pytest.mark.gpu

T = pytest.importorskip("transformer_fwd_bwd_amd")
from transformer_fwd_bwd_amd import gpt as G  # noqa: E402


def oracle_step(params_np, loss_fn, lr=1e-3, wd=0.01):
    P = M.as_tensors(params_np)
    loss, logits = loss_fn(P)
    loss.backward()
    grads = {k: t.grad.copy() for k, t in P.items()}
    opt = OPT.AdamW(list(P.values()), lr=lr, weight_decay=wd)
    opt.step()
    return loss.item(), logits.data, grads, {k: t.data for k, t in P.items()}


def test_tiny_mlp_step_and_gpu_gradcheck(ctx):
    params, x, y = S.tiny_mlp()
    ctx.set_precision("fp32")
    m = G.TinyMlp(ctx, params)
    xt = ctx.tensor(x.shape, x)
    opt = T.AdamW(m.param_list, lr=1e-3, weight_decay=0.01)
    loss, logits = m.loss(xt, y)
    opt.zero_grad()
    ctx.backward(loss)
    gl, glog = loss.item(), logits.numpy()
    ggrads = {k: m.P[k].grad() for k in m.names}
    opt.step()
    gnew = {k: m.P[k].numpy() for k in m.names}
    ctx.tape_reset()

    rl, rlog, rgrads, _ = oracle_step(params, lambda P: M.tiny_mlp_loss(P, x, y))
    assert abs(gl - rl) / max(abs(rl), 1) <= 1e-5
    assert_close(glog, rlog, FWD_TOL["fp32"], "logits")
    for k in m.names:
        assert_close(ggrads[k], rgrads[k], GRAD_TOL["fp32"], "grad " + k)
    # AdamW from the GPU's gradients (teacher forcing: near-zero gradients would
    # otherwise let rounding flip the sign of a whole lr-sized step)
    P = M.as_tensors(params)
    for k in m.names:
        P[k].grad = ggrads[k].astype(np.float64)
    OPT.AdamW([P[k] for k in m.names], lr=1e-3, weight_decay=0.01).step()
    for k in m.names:
        assert_close(gnew[k], P[k].data, 1e-4, "param " + k)

    # the pages' gradient check on the GPU: float32, h = 0.01, norm-wise relative error < 1e-3
    h = np.float32(0.01)
    cur = {k: m.P[k].numpy() for k in m.names}
    ctx.zero_grad(m.param_list)
    loss, _ = m.loss(xt, y)
    ctx.backward(loss)
    analytic = {k: m.P[k].grad() for k in m.names}
    ctx.tape_reset()
    ctx.set_grad_enabled(False)
    worst = 0.0
    for k in m.names:
        base = cur[k].copy()
        flat = base.reshape(-1)
        num = np.zeros_like(flat)
        for i in range(flat.size):
            old = flat[i]
            flat[i] = old + h
            m.P[k].write(base)
            lp = m.loss(xt, y)[0].item()
            flat[i] = old - h
            m.P[k].write(base)
            lm = m.loss(xt, y)[0].item()
            flat[i] = old
            ctx.tape_reset()
            num[i] = np.float32(lp - lm) / (np.float32(2) * h)
        m.P[k].write(base)
        a = analytic[k].reshape(-1).astype(np.float64)
        rel = np.linalg.norm(a - num) / (np.linalg.norm(a) + np.linalg.norm(num))
        worst = max(worst, rel)
    ctx.set_grad_enabled(True)
    assert worst < 1e-3, worst
    opt.close()
    xt.release()
    for t in m.param_list:
        t.release()


def test_char_mlp_100_steps_teacher_forced(ctx):
    params = S.char_mlp()
    ctx.set_precision("fp32")
    m = G.CharMlp(ctx, params)
    opt = T.AdamW(m.param_list, lr=1e-3, weight_decay=0.01)
    oP = M.as_tensors(params)
    oopt = OPT.AdamW([oP[k] for k in m.names], lr=1e-3, weight_decay=0.01)
    first = last = None
    for step in range(100):
        ctx_ids, tgt = S.char_mlp_batch(step)
        cur = {k: m.P[k].numpy() for k in m.names}
        # (i) gradients from identical parameters and batch
        loss, _ = m.loss(ctx_ids, tgt)
        opt.zero_grad()
        ctx.backward(loss)
        gl = loss.item()
        ggr = {k: m.P[k].grad() for k in m.names}
        for k in m.names:
            oP[k].data = cur[k].astype(np.float64)
            oP[k].grad = None
        rl, _ = M.char_mlp_loss(oP, ctx_ids, tgt)
        rl.backward()
        assert abs(gl - rl.item()) / max(abs(rl.item()), 1) <= 1e-5, step
        for k in m.names:
            assert_close(ggr[k], oP[k].grad, GRAD_TOL["fp32"], f"step {step} grad {k}")
        # (ii) the update, from the GPU's gradients
        opt.step()
        for k in m.names:
            oP[k].grad = ggr[k].astype(np.float64)
        oopt.step()
        for k in m.names:
            assert_close(m.P[k].numpy(), oP[k].data, 1e-4, f"step {step} param {k}")
        ctx.tape_reset()
        first = gl if first is None else first
        last = gl
    assert last < first          # it learns the (random) next-id statistics a little
    opt.close()
    for t in m.param_list:
        t.release()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_tiny_gpt_step(ctx, prec):
    s, params, ids = S.tiny_gpt()
    ctx.set_precision(prec)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    opt = T.AdamW(model.param_list, lr=1e-3, weight_decay=0.01)
    inputs, targets = G.split_ids(ids)
    loss, logits = model.loss(inputs, targets)
    opt.zero_grad()
    ctx.backward(loss)
    gl, glog = loss.item(), logits.numpy()
    ggr = {k: model.P[k].grad() for k in model.names}
    opt.step()
    gnew = {k: model.P[k].numpy() for k in model.names}
    ctx.tape_reset()

    rl, rlog, rgr, _ = oracle_step(params, lambda P: M.gpt_loss(P, ids, s.n_layer, s.n_head))
    tol_f, tol_g = FWD_TOL[prec], GRAD_TOL[prec]
    assert abs(gl - rl) / max(abs(rl), 1) <= tol_f
    assert_close(glog, rlog.reshape(glog.shape), tol_f, "logits")
    for k in model.names:
        assert_close(ggr[k], rgr[k], tol_g, "grad " + k)
    # the update from the GPU's own gradients (teacher forcing)
    P = M.as_tensors(params)
    for k in model.names:
        P[k].grad = ggr[k].astype(np.float64)
    OPT.AdamW([P[k] for k in model.names], lr=1e-3, weight_decay=0.01).step()
    for k in model.names:
        assert_close(gnew[k], P[k].data, 1e-4, "param " + k)
    opt.close()
    for t in model.param_list:
        t.release()
    ctx.set_precision("fp32")


@pytest.mark.parametrize("adam", [False, True])
def test_circle_classifier_trains_like_the_oracle(ctx, adam):
    """[Autograd-1, "Training loop"]: the 2 -> 16 (tanh) -> 2 classifier of the circle
    x^2 + y^2 < 0.5 trained for 500 steps on the GPU with SGD or AdamW (lr 0.05, no
    weight decay), from the same seeded start as the oracle run: the losses follow the
    oracle's trajectory (float32 against float64 over 500 steps), and AdamW ends well
    under SGD with the points separated."""
    from oracle import optim as OPT
    rng = S.rng_for(11)
    xs = rng.uniform(-1, 1, size=(256, 2)).astype(np.float32)
    ys = ((xs.astype(np.float64) ** 2).sum(1) < 0.5).astype(np.int32)
    r = S.rng_for(12)
    init = [(r.standard_normal((2, 16)) * 0.5).astype(np.float32), np.zeros(16, np.float32),
            (r.standard_normal((16, 2)) * 0.5).astype(np.float32), np.zeros(2, np.float32)]

    # oracle (float64) from the float32 start
    P = [E.Tensor(a.astype(np.float64)) for a in init]
    oopt = OPT.AdamW(P, lr=0.05, weight_decay=0.0) if adam else OPT.SGD(P, lr=0.05)
    X = E.Tensor(xs.astype(np.float64))
    ref = []
    for _ in range(500):
        logits = E.add(E.matmul(E.tanh(E.add(E.matmul(X, P[0]), P[1])), P[2]), P[3])
        loss = E.softmax_cross_entropy(logits, ys)
        oopt.zero_grad()
        loss.backward()
        oopt.step()
        ref.append(loss.item())

    ctx.set_precision("fp32")
    ts = [ctx.tensor(a.shape, a, param=True) for a in init]
    xt = ctx.tensor(xs.shape, xs)
    gopt = T.AdamW(ts, lr=0.05, weight_decay=0.0) if adam else None
    got = []
    for _ in range(500):
        logits = T.linear(T.tanh(T.linear(xt, ts[0], ts[1])), ts[2], ts[3])
        loss = T.softmax_cross_entropy(logits, ys)
        ctx.zero_grad(ts)
        ctx.backward(loss)
        if adam:
            gopt.step()
        else:
            T.sgd_step(ts, 0.05)
        got.append(loss.item())
        ctx.tape_reset()
    pred = T.linear(T.tanh(T.linear(xt, ts[0], ts[1])), ts[2], ts[3]).numpy().argmax(1)
    ctx.tape_reset()
    for t in ts + [xt]:
        t.release()
    got, ref = np.array(got), np.array(ref)
    assert np.max(np.abs(got - ref) / np.maximum(ref, 1e-3)) < 2e-2, "loss trajectory"
    if adam:
        assert got[-1] < 0.1 and (pred == ys).mean() > 0.97


def test_small_gpt_whole_model_gpu_gradcheck(ctx):
    """The pages' gradient check applied to a whole small GPT on the GPU ([Autograd-1,
    "Gradient check"], and its note that the same check runs over a complete small GPT
    with every layer): every number of every parameter tensor (28, laid out as GPT-2's 148) is
    moved by +-h = 0.01, the float32 central difference of the GPU's own loss is compared
    with the analytic gradient, and the norm-wise relative error |a - n| / (|a| + |n|)
    must stay below 1e-3 per tensor.  The model is small enough for one forward per
    number (vocab 16, 16 channels, 2 heads, 2 blocks, 8 positions, batch 2: 6,976
    numbers); its weights are drawn wider than GPT-2's (std 0.2, random LayerNorm gains,
    shifts and biases) so that a step of h moves the float32 loss by far more than its
    rounding."""
    shape = S.GptShape(vocab=16, n_positions=8, n_layer=2, n_head=2, n_embd=16)
    params = S.gpt_params(shape, 90, std=0.2)
    rng = S.rng_for(91)
    for k in params:
        if params[k].ndim == 1:
            params[k] = (params[k] + 0.1 * rng.standard_normal(params[k].shape)).astype(np.float32)
    ids = S.random_ids(92, (2, shape.n_positions + 1), shape.vocab)
    ctx.set_precision("fp32")
    model = G.Gpt(ctx, shape.n_layer, shape.n_head, params)
    inputs, targets = G.split_ids(ids)
    ctx.zero_grad(model.param_list)
    loss, _ = model.loss(inputs, targets)
    ctx.backward(loss)
    analytic = {k: model.P[k].grad() for k in model.names}
    ctx.tape_reset()
    ctx.set_grad_enabled(False)
    h = np.float32(0.01)
    worst, worst_k = 0.0, None
    try:
        for k in model.names:
            base = params[k].copy()
            flat = base.reshape(-1)
            num = np.zeros(flat.size, np.float32)
            for i in range(flat.size):
                old = flat[i]
                flat[i] = old + h
                model.P[k].write(base)
                lp = np.float32(model.loss(inputs, targets)[0].item())
                ctx.tape_reset()
                flat[i] = old - h
                model.P[k].write(base)
                lm = np.float32(model.loss(inputs, targets)[0].item())
                ctx.tape_reset()
                flat[i] = old
                num[i] = (lp - lm) / (np.float32(2) * h)
            model.P[k].write(base)
            a = analytic[k].reshape(-1).astype(np.float64)
            n = num.astype(np.float64)
            den = np.linalg.norm(a) + np.linalg.norm(n)
            rel = np.linalg.norm(a - n) / den if den > 0 else 0.0
            if rel > worst:
                worst, worst_k = rel, k
    finally:
        ctx.set_grad_enabled(True)
    print(f"whole-model gradient check: worst relative error {worst:.2e} ({worst_k}) over {len(model.names)} tensors")
    assert len(model.names) == 4 + 12 * shape.n_layer
    assert worst < 1e-3, (worst, worst_k)
    for t in model.param_list:
        t.release()
