"""Pins of the oracle's scalar layer, finite differences and gradient check
against values the pages print (fixtures under tests/golden/, each cited)."""
import math

import numpy as np
import pytest

from oracle import engine as E
from oracle import gradcheck as G
from oracle.scalar import Dual, Value, scalar_gradient_check


def sig3(x):
    """Round to 3 significant digits, the precision of the pages' E2 format."""
    return float(f"{x:.2E}")


def test_derivative_table_float32(golden):
    fx = golden("autograd1_derivative.json")
    f = lambda x: x * x
    x = np.float32(fx["x"])
    for row in fx["rows"]:
        h = np.float32(row["h"])
        fwd = G.forward_difference(f, x, h)
        cen = G.central_difference(f, x, h)
        assert isinstance(fwd, np.float32) and isinstance(cen, np.float32)
        assert f"{fwd:.4f}" == row["forward"]
        assert f"{cen:.4f}" == row["central"]


def test_tiny_graph(golden):
    fx = golden("autograd1_tinygraph.json")
    t = {k: E.Tensor(np.array([v], np.float32)) for k, v in fx["inputs"].items()}
    z = E.add(E.mul(t["w"], t["x"]), t["b"])
    L = E.mul(z, z)
    L.backward()
    assert z.item() == fx["forward"]["z"] and L.item() == fx["forward"]["L"]
    got = {"dL/dz": z.grad[0], "dL/dw": t["w"].grad[0], "dL/dx": t["x"].grad[0], "dL/db": t["b"].grad[0]}
    assert got == fx["backward"]
    h = np.float32(fx["numeric"]["h"])
    Lw = lambda wv: (wv * np.float32(3) + np.float32(1)) * (wv * np.float32(3) + np.float32(1))
    assert f"{G.central_difference(Lw, np.float32(2), h):.3f}" == fx["numeric"]["dL/dw"]


def test_break_it_on_purpose(golden):
    fx = golden("autograd1_break_it.json")
    z = E.Tensor(np.array([fx["z"]], np.float32))
    for row, mul in zip(fx["rows"], (E.mul, E.mul_assign_wrong)):
        z.zero_grad()
        mul(z, z).backward()
        _, rel = G.run(lambda: mul(z, z), [z], h=0.01)
        assert z.grad[0] == row["grad"]
        assert sig3(rel) == float(row["max_rel"].replace("E-00", "E-0"))
        assert (rel < fx["threshold"]) == (row["verdict"] == "OK")


def test_sin_x2_reverse_and_forward(golden):
    fx = golden("chainrule_worked_examples.json")["sin_x2"]
    x = Value(fx["x"])
    a = x ** 2
    y = a.sin()
    y.backward()
    assert round(x.grad, 3) == fx["dy_dx_printed"]
    assert round(a.grad, 3) == fx["dy_da_printed"]
    d = (Dual(fx["x"], 1.0) ** 2).sin()
    assert abs(d.deriv - x.grad) < 1e-12
    # closed form 2x cos(x^2)
    assert abs(x.grad - 4 * math.cos(4.0)) < 1e-12


def test_chainrule_examples(golden):
    fx = golden("chainrule_worked_examples.json")
    x = Value(fx["poly"]["x"])
    y = x ** 2 + 3 * x + 1
    y.backward()
    assert x.grad == fx["poly"]["grad"]

    r = fx["relu_product"]
    x1, x2 = Value(r["x1"]), Value(r["x2"])
    y = (x1 * x2 + Value(1.0)).relu()
    y.backward()
    assert (y.data, x1.grad, x2.grad) == (r["y"], r["dy_dx1"], r["dy_dx2"])

    r = fx["relu_abc"]
    a, b, c = Value(r["a"]), Value(r["b"]), Value(r["c"])
    f = (a * b + c).relu()
    f.backward()
    assert (f.data, a.grad, b.grad, c.grad) == (r["f"], r["df_da"], r["df_db"], r["df_dc"])

    x = Value(fx["cube"]["x"])
    (x ** 3).backward()
    assert x.grad == fx["cube"]["grad"]

    for t in fx["tanh_prime"]:
        x = Value(t["x"])
        x.tanh().backward()
        assert round(x.grad, t["decimals"]) == t["value"]
        num = (math.tanh(t["x"] + 1e-6) - math.tanh(t["x"] - 1e-6)) / 2e-6
        assert abs(num - x.grad) < 1e-8

    gc = fx["gradient_check"]
    ad, num, diff = scalar_gradient_check(lambda v: (v ** 3 + v * 2 + 1).tanh(), gc["x"], gc["h"])
    assert diff < gc["max_diff"]


def test_relu_negative_branch_zero_grads():
    # exercise 3 of the chain-rule page: a negative relu input zeroes all five gradients
    w1, x1, w2, x2, b = (Value(v) for v in (1.0, -2.0, 0.5, 1.0, -1.0))
    y = (w1 * x1 + w2 * x2 + b).relu()
    y.backward()
    assert [v.grad for v in (w1, x1, w2, x2, b)] == [0.0] * 5


def test_dual_matches_reverse_on_composite():
    f_rev = lambda v: (v ** 3 + v * 2 + 1).tanh()
    x = Value(0.7)
    f_rev(x).backward()
    d = ((Dual(0.7, 1.0) ** 3) + Dual(0.7, 1.0) * 2 + 1).tanh()
    assert abs(d.deriv - x.grad) < 1e-12


def test_planted_mistake_in_scalar_rule_is_caught(monkeypatch):
    # a wrong tanh rule (g * y instead of g * (1 - y^2)) must fail the scalar check
    def bad_tanh(self):
        t = math.tanh(self.data)
        return Value.node(t, "tanh", (self, t))
    monkeypatch.setattr(Value, "tanh", bad_tanh)
    _, _, diff = scalar_gradient_check(lambda v: (v ** 3 + v * 2 + 1).tanh(), 0.5)
    assert diff > 1e-3
