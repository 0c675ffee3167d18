"""Scalar automatic differentiation: reverse mode (Value) and forward mode (Dual).

Test infrastructure only.  Reverse mode follows [ChainRule, steps 1-4]: every
operation makes a node that remembers its inputs and a closure adding
(local derivative) x (upstream gradient) into each input; backward() orders the
nodes depth-first, seeds dy/dy = 1 and calls the closures in reverse.  Forward
mode follows [ChainRule, §"Dual numbers for forward mode"]: a pair
(value, derivative) with the sum, product and sine rules.  sin/cos are added to
both so that the page's worked example d/dx sin(x^2) can be computed.
"""
from __future__ import annotations

import math


class Value:
    def __init__(self, data, children=(), op=""):
        self.data = float(data)
        self.grad = 0.0
        self._backward = lambda: None
        self._prev = tuple(children)
        self._op = op

    @staticmethod
    def _lift(o):
        return o if isinstance(o, Value) else Value(o)

    def __add__(self, other):
        other = Value._lift(other)
        out = Value(self.data + other.data, (self, other), "+")

        def bw():
            self.grad += out.grad
            other.grad += out.grad
        out._backward = bw
        return out

    def __mul__(self, other):
        other = Value._lift(other)
        out = Value(self.data * other.data, (self, other), "*")

        def bw():
            self.grad += other.data * out.grad
            other.grad += self.data * out.grad
        out._backward = bw
        return out

    def __pow__(self, n):
        out = Value(self.data ** n, (self,), f"**{n}")

        def bw():
            self.grad += n * self.data ** (n - 1) * out.grad
        out._backward = bw
        return out

    def _unary(self, value, local, op):
        out = Value(value, (self,), op)

        def bw():
            self.grad += local * out.grad
        out._backward = bw
        return out

    def relu(self):
        return self._unary(max(0.0, self.data), 1.0 if self.data > 0 else 0.0, "relu")

    def exp(self):
        e = math.exp(self.data)
        return self._unary(e, e, "exp")

    def log(self):
        return self._unary(math.log(self.data), 1.0 / self.data, "log")

    def tanh(self):
        t = math.tanh(self.data)
        return self._unary(t, 1 - t * t, "tanh")

    def sin(self):
        return self._unary(math.sin(self.data), math.cos(self.data), "sin")

    def cos(self):
        return self._unary(math.cos(self.data), -math.sin(self.data), "cos")

    # composite operations get their rules from the primitives
    def __neg__(self):
        return self * -1

    def __sub__(self, other):
        return self + (-Value._lift(other))

    def __radd__(self, other):
        return self + other

    def __rmul__(self, other):
        return self * other

    def __rsub__(self, other):
        return Value._lift(other) + (-self)

    def __truediv__(self, other):
        return self * (Value._lift(other) ** -1)

    def backward(self):
        topo, seen = [], set()

        def build(v):
            if id(v) not in seen:
                seen.add(id(v))
                for c in v._prev:
                    build(c)
                topo.append(v)
        build(self)
        self.grad = 1.0
        for v in reversed(topo):
            v._backward()


class Dual:
    """a + a' eps with eps^2 = 0."""

    def __init__(self, value, deriv=0.0):
        self.value = float(value)
        self.deriv = float(deriv)

    @staticmethod
    def _lift(o):
        return o if isinstance(o, Dual) else Dual(o, 0.0)

    def __add__(self, o):
        o = Dual._lift(o)
        return Dual(self.value + o.value, self.deriv + o.deriv)

    __radd__ = __add__

    def __mul__(self, o):
        o = Dual._lift(o)
        return Dual(self.value * o.value, self.deriv * o.value + self.value * o.deriv)

    __rmul__ = __mul__

    def __pow__(self, n):
        return Dual(self.value ** n, n * self.value ** (n - 1) * self.deriv)

    def sin(self):
        return Dual(math.sin(self.value), math.cos(self.value) * self.deriv)

    def tanh(self):
        t = math.tanh(self.value)
        return Dual(t, (1 - t * t) * self.deriv)


def scalar_gradient_check(build_expr, x_val, h=1e-7):
    """[ChainRule, step 6]: reverse-mode gradient vs central difference in double."""
    x = Value(x_val)
    y = build_expr(x)
    y.backward()
    ad = x.grad
    num = (build_expr(Value(x_val + h)).data - build_expr(Value(x_val - h)).data) / (2 * h)
    return ad, num, abs(ad - num)
