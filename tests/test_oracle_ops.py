"""Pins of the oracle's tensor ops against brute force, closed forms, finite
differences and library routines -- never against a retyped copy of the same
formula.  CPU only."""
import math

import numpy as np
import pytest

from oracle import engine as E
from oracle import gradcheck as G
from oracle import ops as O
from synthetic import random_array, random_ids


def T64(a):
    return E.Tensor(np.array(a, dtype=np.float64))


# --------------------------------------------------------------------------
# Finite-difference check of every backward rule (float64, h = 1e-5)
# --------------------------------------------------------------------------
def _R(shape, seed=99):
    return random_array(seed, shape, dtype=np.float64)


def _op_cases():
    r = lambda s, seed, sc=1.0: T64(random_array(seed, s, sc))
    cases = {}
    a, b = r((3, 4), 1), r((3, 4), 2)
    cases["Add"] = (lambda: E.add(a, b), [a, b], (3, 4))
    a2, bias = r((2, 3, 4), 3), r((4,), 4)
    cases["Add (broadcast bias)"] = (lambda: E.add(a2, bias), [a2, bias], (2, 3, 4))
    m1, m2 = r((3, 4), 5), r((3, 4), 6)
    cases["Mul"] = (lambda: E.mul(m1, m2), [m1, m2], (3, 4))
    s1 = r((3, 4), 7)
    cases["Scale"] = (lambda: E.scale(s1, 0.37), [s1], (3, 4))
    x, w = r((2, 3, 5), 8), r((5, 4), 9)
    cases["MatMul"] = (lambda: E.matmul(x, w), [x, w], (2, 3, 4))
    xt, wt = r((3, 5), 10), r((6, 5), 11)
    cases["MatMulT"] = (lambda: E.matmul_t(xt, wt), [xt, wt], (3, 6))
    th = r((3, 4), 12)
    cases["Tanh"] = (lambda: E.tanh(th), [th], (3, 4))
    ge = r((3, 4), 13, 2.0)
    cases["Gelu"] = (lambda: E.gelu(ge), [ge], (3, 4))
    rs = r((3, 4), 14)
    cases["Reshape"] = (lambda: E.reshape(rs, (2, 6)), [rs], (2, 6))
    tab = r((5, 3), 15)
    ids = np.array([1, 4, 1, 0, 3, 1])
    cases["Embedding"] = (lambda: E.embedding(tab, ids, 2), [tab], (2, 3, 3))
    lx, lg, lb = r((3, 6), 16), r((6,), 17), r((6,), 18)
    cases["LayerNorm"] = (lambda: E.layernorm(lx, lg, lb), [lx, lg, lb], (3, 6))
    ba, bb = r((2, 3, 4), 19), r((2, 5, 4), 20)
    cases["BatchMatMulT"] = (lambda: E.batch_matmul_t(ba, bb), [ba, bb], (2, 3, 5))
    bc, bd = r((2, 3, 4), 21), r((2, 4, 5), 22)
    cases["BatchMatMul"] = (lambda: E.batch_matmul(bc, bd), [bc, bd], (2, 3, 5))
    cs = r((2, 2, 4, 4), 23)
    cases["CausalSoftmax"] = (lambda: E.causal_softmax(cs), [cs], (2, 2, 4, 4))
    nx = r((2, 3, 9), 24)
    cases["Narrow"] = (lambda: E.narrow(nx, 3, 4), [nx], (2, 3, 4))
    sx = r((2, 3, 8), 25)
    cases["SplitHeads"] = (lambda: E.split_heads(sx, 2), [sx], (2, 2, 3, 4))
    mx = r((2, 2, 3, 4), 26)
    cases["MergeHeads"] = (lambda: E.merge_heads(mx), [mx], (2, 3, 8))
    return cases


@pytest.mark.parametrize("name", list(_op_cases().keys()))
def test_backward_rule_matches_central_difference_fp64(name):
    fn, inputs, out_shape = _op_cases()[name]
    loss = G.projected(fn, _R(out_shape))
    _, rel = G.run(loss, inputs, h=1e-5)
    assert rel < 1e-8, (name, rel)


def test_softmax_ce_backward_fd_fp64():
    lg = T64(random_array(30, (4, 7)))
    tg = np.array([0, 6, 3, 3])
    _, rel = G.run(lambda: E.softmax_cross_entropy(lg, tg), [lg], h=1e-5)
    assert rel < 1e-8


def test_pages_op_table_in_float32(golden):
    """The pages' own check (float, h = 0.01): every op passes with a relative
    error well below the threshold, of the order the printed table shows."""
    fx = golden("autograd1_gradcheck_ops.json")
    cases = _op_cases()
    for name in fx["max_rel"]:
        if name == "SoftmaxCrossEntropy":
            lg = E.Tensor(random_array(30, (4, 7)))
            _, rel = G.run(lambda: E.softmax_cross_entropy(lg, [0, 6, 3, 3]), [lg], h=fx["h"])
        else:
            fn, inputs, out_shape = cases[name]
            for t in inputs:
                t.data = t.data.astype(np.float32)
                t.grad = None
            Rt = random_array(99, out_shape)
            _, rel = G.run(G.projected(fn, Rt), inputs, h=fx["h"])
        assert rel < fx["threshold"], (name, rel)
        assert rel < 100 * max(fx["max_rel"][name], 1e-5), (name, rel)


# --------------------------------------------------------------------------
# Planted mistakes must be caught by the checks (the pages' negative test)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("target,bad", [
    ("tanh_bwd", lambda g, y: g * y),                                   # the pages' exercise
    ("matmul_bwd", lambda g, x, w: ((g.reshape(-1, g.shape[-1]) @ w.T).reshape(x.shape),
                                    g.reshape(-1, g.shape[-1]).T @ x.reshape(-1, x.shape[-1]))),  # dw transposed
    ("layernorm_bwd", lambda g, x, gm, mu, rs: (rs * (g * gm - (g * gm).mean(-1, keepdims=True)),
                                                (g * (x - mu) * rs).sum(0), g.sum(0))),
    ("gelu_bwd", lambda g, x: g * 0.5 * (1 + np.tanh(O.GELU_C * x))),
    ("causal_softmax_bwd", lambda g, p: p * g),
])
def test_planted_backward_mistakes_fail(monkeypatch, target, bad):
    monkeypatch.setattr(O, target, bad)
    cases = _op_cases()
    name = {"tanh_bwd": "Tanh", "matmul_bwd": "MatMul", "layernorm_bwd": "LayerNorm",
            "gelu_bwd": "Gelu", "causal_softmax_bwd": "CausalSoftmax"}[target]
    fn, inputs, out_shape = cases[name]
    if target == "matmul_bwd":
        # square weight so the transposed gradient has the right shape but wrong values
        x, w = T64(random_array(8, (2, 3, 4))), T64(random_array(9, (4, 4)))
        fn, inputs, out_shape = (lambda: E.matmul(x, w)), [x, w], (2, 3, 4)
    _, rel = G.run(G.projected(fn, _R(out_shape)), inputs, h=1e-5)
    assert rel > 1e-3


def test_assign_instead_of_add_is_caught_on_residual():
    x = T64(random_array(40, (3, 4)))
    w = T64(random_array(41, (4, 4)))
    good = lambda: E.sum_all(E.mul(E.add(E.matmul(x, w), x), E.add(E.matmul(x, w), x)))
    _, rel = G.run(good, [x, w], h=1e-5)
    assert rel < 1e-8
    bad = lambda: E.sum_all(E.mul_assign_wrong(E.add(E.matmul(x, w), x), E.add(E.matmul(x, w), x)))
    # with two distinct (but equal-valued) branches the assignment is harmless...
    _, rel = G.run(bad, [x, w], h=1e-5)
    assert rel < 1e-8
    # ...but with one tensor used twice it loses half of the gradient
    y = lambda: E.add(E.matmul(x, w), x)
    bad2 = lambda: (lambda t: E.sum_all(E.mul_assign_wrong(t, t)))(y())
    _, rel = G.run(bad2, [x, w], h=1e-5)
    assert rel > 0.1


# --------------------------------------------------------------------------
# MatMul family: brute force and textbook special cases
# --------------------------------------------------------------------------
def _triple_loop(a, b):
    n, k = a.shape
    m = b.shape[1]
    c = [[0.0] * m for _ in range(n)]
    for i in range(n):
        for j in range(m):
            s = 0.0
            for p in range(k):
                s += float(a[i, p]) * float(b[p, j])
            c[i][j] = s
    return np.array(c)


def test_matmul_family_brute_force():
    a = random_array(50, (5, 7), dtype=np.float64)
    b = random_array(51, (7, 3), dtype=np.float64)
    assert np.allclose(O.matmul_fwd(a, b), _triple_loop(a, b), rtol=1e-13, atol=1e-13)
    bt = np.ascontiguousarray(b.T)
    assert np.allclose(O.matmul_t_fwd(a, bt), _triple_loop(a, b), rtol=1e-13, atol=1e-13)
    g = random_array(52, (5, 3), dtype=np.float64)
    dx, dw = O.matmul_bwd(g, a, b)
    assert np.allclose(dx, _triple_loop(g, bt), atol=1e-13)
    assert np.allclose(dw, _triple_loop(np.ascontiguousarray(a.T), g), atol=1e-13)
    dx2, dw2 = O.matmul_t_bwd(g, a, bt)
    assert np.allclose(dx2, dx, atol=1e-13) and np.allclose(dw2, dw.T, atol=1e-13)
    A = random_array(53, (2, 4, 3), dtype=np.float64)
    B = random_array(54, (2, 3, 5), dtype=np.float64)
    Cb = O.batch_matmul_fwd(A, B)
    Ct = O.batch_matmul_t_fwd(A, np.ascontiguousarray(np.swapaxes(B, 1, 2)))
    for z in range(2):
        assert np.allclose(Cb[z], _triple_loop(A[z], B[z]), atol=1e-13)
        assert np.allclose(Ct[z], Cb[z], atol=1e-13)


def test_matmul_identity_gives_input_back():
    x = random_array(55, (6, 8), dtype=np.float64)
    assert np.array_equal(O.matmul_fwd(x, np.eye(8)), x)
    assert np.array_equal(O.matmul_t_fwd(x, np.eye(8)), x)


# --------------------------------------------------------------------------
# Softmax family: closed forms and invariants
# --------------------------------------------------------------------------
@pytest.mark.parametrize("V", [4, 64, 50257])
def test_ce_uniform_logits_gives_log_v(V):
    n = 3
    loss, p = O.softmax_ce_fwd(np.zeros((n, V)), np.array([0, V - 1, V // 2]))
    assert abs(loss[0] - math.log(V)) < 1e-12
    d = O.softmax_ce_bwd(np.array([1.0]), p, np.array([0, V - 1, V // 2]))
    assert abs(d[0, 1] - 1 / V / n) < 1e-15 and abs(d[0, 0] - (1 / V - 1) / n) < 1e-15


def test_ce_rows_and_grad_rows():
    L = random_array(60, (5, 11), 3.0, dtype=np.float64)
    t = random_ids(61, (5,), 11)
    loss, p = O.softmax_ce_fwd(L, t)
    assert np.allclose(p.sum(1), 1, atol=1e-14)
    d = O.softmax_ce_bwd(np.array([1.0]), p, t)
    assert np.allclose(d.sum(1), 0, atol=1e-15)
    # loss by the textbook log-sum-exp identity
    lse = np.log(np.exp(L).sum(1))
    assert abs(loss[0] - (lse - L[np.arange(5), t]).mean()) < 1e-12
    # shift invariance
    loss2, _ = O.softmax_ce_fwd(L + 1000.0, t)
    assert abs(loss2[0] - loss[0]) < 1e-9


def test_causal_softmax_structure():
    T = 5
    s = random_array(62, (2, 3, T, T), dtype=np.float64)
    p = O.causal_softmax_fwd(s)
    rows = p.reshape(-1, T)
    for r in range(rows.shape[0]):
        vis = r % T + 1
        assert np.count_nonzero(rows[r]) == vis
        assert np.all(rows[r, vis:] == 0)
        assert abs(rows[r].sum() - 1) < 1e-14
        # the visible part is a plain softmax of the visible scores
        e = np.exp(s.reshape(-1, T)[r, :vis])
        assert np.allclose(rows[r, :vis], e / e.sum(), atol=1e-15)
    assert np.all(rows[::T, 0] == 1.0)


def test_attention_special_cases():
    # T = 1 returns V exactly; equal keys give the mean of visible values
    v = random_array(63, (3, 1, 4), dtype=np.float64)
    q = random_array(64, (3, 1, 4), dtype=np.float64)
    k = random_array(65, (3, 1, 4), dtype=np.float64)
    p = O.causal_softmax_fwd(O.batch_matmul_t_fwd(q, k) / 2.0)
    assert np.array_equal(O.batch_matmul_fwd(p, v), v)
    T = 6
    kk = np.tile(random_array(66, (1, 1, 4), dtype=np.float64), (2, T, 1))
    qq = random_array(67, (2, T, 4), dtype=np.float64)
    vv = random_array(68, (2, T, 4), dtype=np.float64)
    o = O.batch_matmul_fwd(O.causal_softmax_fwd(O.batch_matmul_t_fwd(qq, kk)), vv)
    for t in range(T):
        assert np.allclose(o[:, t], vv[:, :t + 1].mean(1), atol=1e-14)


# --------------------------------------------------------------------------
# LayerNorm, GELU, Embedding
# --------------------------------------------------------------------------
def test_layernorm_moments_and_orthogonality():
    x = random_array(70, (7, 32), 3.0, dtype=np.float64) + 5.0
    y, mu, rstd = O.layernorm_fwd(x, np.ones(32), np.zeros(32))
    var = x.var(axis=1)
    assert np.allclose(y.mean(1), 0, atol=1e-14)
    assert np.allclose(y.var(1), var / (var + O.LN_EPS), atol=1e-13)
    g = random_array(71, (7, 32), dtype=np.float64)
    # with eps = 0 the gradient rows are orthogonal to 1 and to xhat exactly
    y, mu, rstd = O.layernorm_fwd(x, np.ones(32), np.zeros(32), eps=0.0)
    dx, _, _ = O.layernorm_bwd(g, x, np.ones(32), mu, rstd)
    xhat = (x - mu) * rstd
    assert np.allclose(dx.sum(1), 0, atol=1e-12)
    assert np.allclose((dx * xhat).sum(1), 0, atol=1e-12)


def test_gelu_tanh_vs_erf_form():
    """The tanh form approximates x * Phi(x) (math.erf) closely but not exactly
    ([GPT2-4, §"Common mistakes"]: the exact form is a different function).

    Pins that do not restate the formula:
    * its largest deviation from x * Phi(x) on [-8, 8] lies in (4e-4, 5e-4).  The
      published constants give 4.73e-4; a slip in either constant moves it out of
      that band (sqrt(2/pi) -> 0.8 gives 6.4e-4; 0.044715 -> 0.045 gives 5.6e-4,
      -> 0.04 gives 2.9e-3, a dropped cubic term gives 3.4e-2);
    * at 0 the tanh form must share the exact function's first two derivatives:
      d/dx [x Phi(x)] = Phi(0) = 1/2 and d2/dx2 [x Phi(x)] = 2 phi(0) = sqrt(2/pi)
      (the constant in front of the bracket is chosen for exactly this)."""
    xs = np.linspace(-8, 8, 32001)
    exact = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in xs])
    d = np.abs(O.gelu_fwd(xs) - exact)
    assert 4e-4 < d.max() < 5e-4, d.max()
    h = 1e-3
    g = lambda v: O.gelu_fwd(np.array([v], np.float64))[0]
    d1 = (g(h) - g(-h)) / (2 * h)
    d2 = (g(h) - 2 * g(0.0) + g(-h)) / (h * h)
    phi0 = 1.0 / math.sqrt(2 * math.pi)
    assert abs(d1 - 0.5) < 1e-9
    assert abs(d2 - 2 * phi0) < 1e-5, (d2, 2 * phi0)
    assert O.gelu_fwd(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu_fwd(np.array([20.0]))[0] - 20.0) < 1e-12
    assert abs(O.gelu_fwd(np.array([-20.0]))[0]) < 1e-12


@pytest.mark.parametrize("const,bad", [("GELU_C", 0.8), ("GELU_A", 0.045), ("GELU_A", 0.0)])
def test_planted_gelu_constant_mistakes_fail(monkeypatch, const, bad):
    monkeypatch.setattr(O, const, bad)
    with pytest.raises(AssertionError):
        test_gelu_tanh_vs_erf_form()


def test_embedding_routing_is_exact():
    table = random_array(80, (9, 5), dtype=np.float32)
    ids = random_ids(81, (4, 6), 9)
    out = O.embedding_fwd(table, ids.reshape(-1), 4)
    assert out.shape == (4, 6, 5)
    for b in range(4):
        for t in range(6):
            assert np.array_equal(out[b, t], table[ids[b, t]])
    d = O.embedding_bwd(np.ones((4, 6, 5), np.float32), ids.reshape(-1), table.shape)
    counts = np.bincount(ids.reshape(-1), minlength=9)
    assert np.array_equal(d, np.repeat(counts[:, None], 5, axis=1).astype(np.float32))
    with pytest.raises(IndexError):
        O.embedding_fwd(table, np.array([9]), 1)


def test_shape_errors_mirror_the_pages():
    with pytest.raises(ValueError):
        O.mul_fwd(np.zeros(3), np.zeros(4))
    with pytest.raises(ValueError):
        O.matmul_fwd(np.zeros((2, 3)), np.zeros((4, 5)))
    with pytest.raises(ValueError):
        O.softmax_ce_fwd(np.zeros((3, 4)), np.zeros(2, np.int32))
    with pytest.raises(ValueError):
        E.sum_all(T64(np.ones(3))).data  # fine
        E.add(T64(np.ones((2, 3))), T64(np.ones((2,))))
    with pytest.raises(ValueError):
        E.tanh(T64(np.ones(3))).backward()


# --------------------------------------------------------------------------
# Tape semantics
# --------------------------------------------------------------------------
def test_leaf_grads_accumulate_until_zero_grad():
    w = T64([2.0])
    x = T64([3.0])
    for k in (1, 2, 3):
        E.mul(w, x).backward()
        assert w.grad[0] == 3.0 * k
    w.zero_grad()
    E.mul(w, x).backward()
    assert w.grad[0] == 3.0


def test_no_grad_records_nothing():
    a = T64([1.0, 2.0])
    with E.no_grad():
        y = E.tanh(a)
    assert y.parents == () and y.backward_rule is None


def test_topological_order_puts_inputs_first():
    a, b = T64([1.0]), T64([2.0])
    z = E.add(E.mul(a, b), b)
    L = E.mul(z, z)
    order = L.topological_order()
    pos = {id(t): i for i, t in enumerate(order)}
    for t in order:
        for p in t.parents:
            assert pos[id(p)] < pos[id(t)]
    assert order[-1] is L
