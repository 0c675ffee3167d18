"""Scalar automatic differentiation: reverse mode (Value) and forward mode (Dual).

Test infrastructure only.

Reverse mode ([ChainRule], the steps that build a scalar engine): every
operation returns a node holding its value and, for each input, the local
partial derivative of the output with respect to that input, evaluated when the
node is made.  No closures are kept: a node is data (value, inputs, partials).
backward() then applies the chain rule over the graph reachable from the output
in an order where a node is finished only after every node that consumes it:
it counts each node's consumers inside that graph and releases a node to the
work list once all of them have passed their gradient down (a consumer-count
sweep, Kahn's algorithm run from the output towards the inputs).  Each input's
gradient receives partial x upstream gradient, added, so a value used twice
collects both contributions.

Subtraction, negation and division are primitives here, each with its own
partials (1 and -1; -1; 1/b and -a/b^2), not compositions of the other rules.

Forward mode ([ChainRule], the section on dual numbers): a pair (value,
derivative) propagated with the sum, product, power, sine and tanh rules.
sin/cos exist in both modes so that the page's worked example d/dx sin(x^2)
can be computed either way.
"""
from __future__ import annotations

import math
from collections import deque


class Value:
    __slots__ = ("data", "grad", "inputs", "partials", "op")

    def __init__(self, data, inputs=(), partials=(), op=""):
        self.data = float(data)
        self.grad = 0.0
        self.inputs = tuple(inputs)       # the nodes this one was computed from
        self.partials = tuple(partials)   # d(self)/d(inputs[i]), fixed at creation
        self.op = op

    # ------------------------------------------------------------ building
    @staticmethod
    def _as_node(o) -> "Value":
        return o if isinstance(o, Value) else Value(o)

    @staticmethod
    def node(value, op, *pairs) -> "Value":
        """A new node from (input, local partial) pairs."""
        return Value(value, tuple(p[0] for p in pairs), tuple(float(p[1]) for p in pairs), op)

    def __add__(self, other):
        b = Value._as_node(other)
        return Value.node(self.data + b.data, "+", (self, 1.0), (b, 1.0))

    def __radd__(self, other):
        return Value._as_node(other).__add__(self)

    def __sub__(self, other):
        b = Value._as_node(other)
        return Value.node(self.data - b.data, "-", (self, 1.0), (b, -1.0))

    def __rsub__(self, other):
        return Value._as_node(other).__sub__(self)

    def __neg__(self):
        return Value.node(-self.data, "neg", (self, -1.0))

    def __mul__(self, other):
        b = Value._as_node(other)
        return Value.node(self.data * b.data, "*", (self, b.data), (b, self.data))

    def __rmul__(self, other):
        return Value._as_node(other).__mul__(self)

    def __truediv__(self, other):
        b = Value._as_node(other)
        q = self.data / b.data
        return Value.node(q, "/", (self, 1.0 / b.data), (b, -q / b.data))

    def __rtruediv__(self, other):
        return Value._as_node(other).__truediv__(self)

    def __pow__(self, n):
        if isinstance(n, Value):
            raise TypeError("only constant exponents")
        return Value.node(self.data ** n, f"^{n}", (self, n * self.data ** (n - 1)))

    def relu(self):
        return Value.node(self.data if self.data > 0 else 0.0, "relu", (self, 1.0 if self.data > 0 else 0.0))

    def exp(self):
        e = math.exp(self.data)
        return Value.node(e, "exp", (self, e))

    def log(self):
        return Value.node(math.log(self.data), "log", (self, 1.0 / self.data))

    def tanh(self):
        t = math.tanh(self.data)
        return Value.node(t, "tanh", (self, 1.0 - t * t))

    def sin(self):
        return Value.node(math.sin(self.data), "sin", (self, math.cos(self.data)))

    def cos(self):
        return Value.node(math.cos(self.data), "cos", (self, -math.sin(self.data)))

    # ------------------------------------------------------------ reverse sweep
    def backward(self):
        # 1. consumers of every node reachable from the output (an explicit stack, no recursion)
        consumers = {id(self): 0}
        nodes = {id(self): self}
        stack = [self]
        while stack:
            v = stack.pop()
            for u in v.inputs:
                k = id(u)
                if k not in nodes:
                    nodes[k] = u
                    consumers[k] = 0
                    stack.append(u)
                consumers[k] += 1
        # 2. chain rule: a node passes its gradient down once all its consumers have
        #    added theirs; its inputs' counters drop and reach zero in turn.
        self.grad = 1.0
        ready = deque([self])
        while ready:
            v = ready.popleft()
            for u, d in zip(v.inputs, v.partials):
                u.grad += d * v.grad
                k = id(u)
                consumers[k] -= 1
                if consumers[k] == 0:
                    ready.append(u)


class Dual:
    """value + deriv * eps with eps^2 = 0."""

    __slots__ = ("value", "deriv")

    def __init__(self, value, deriv=0.0):
        self.value = float(value)
        self.deriv = float(deriv)

    @staticmethod
    def _as_dual(o) -> "Dual":
        return o if isinstance(o, Dual) else Dual(o, 0.0)

    def __add__(self, o):
        o = Dual._as_dual(o)
        return Dual(self.value + o.value, self.deriv + o.deriv)

    __radd__ = __add__

    def __mul__(self, o):
        o = Dual._as_dual(o)
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
    """Reverse-mode gradient of build_expr at x_val against a central difference in
    double ([ChainRule], the gradient-check step); returns (ad, numeric, |ad - numeric|)."""
    x = Value(x_val)
    y = build_expr(x)
    y.backward()
    ad = x.grad
    num = (build_expr(Value(x_val + h)).data - build_expr(Value(x_val - h)).data) / (2 * h)
    return ad, num, abs(ad - num)
