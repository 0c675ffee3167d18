"""Tensor and tape of the oracle: record on forward, replay backward rules in reverse.

Test infrastructure only.  Semantics follow [Autograd-1, §"The Tensor class" and
§"How each op records itself in the graph"]:

* a tensor holds flat data, a gradient created on demand, a shape, the op that
  made it ("leaf" for inputs and parameters), its parents and a backward rule;
* while no_grad is set, ops record nothing;
* backward() starts only from a one-element loss; it orders the graph reachable
  from the loss so that every node comes after its inputs (depth-first), clears
  the gradients of non-leaf nodes, seeds dLoss/dLoss = 1 and runs the rules from
  the end of that order to its start;
* every rule ADDS into its inputs' gradients; leaf gradients are never cleared
  by backward() -- the optimizer's zero_grad clears them.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np

from . import ops as O

_no_grad = [False]


class no_grad:
    """Context manager for inference mode (the pages' NoGrad flag)."""

    def __enter__(self):
        self.old = _no_grad[0]
        _no_grad[0] = True

    def __exit__(self, *exc):
        _no_grad[0] = self.old


class Tensor:
    def __init__(self, data, op: str = "leaf", name: str = ""):
        self.data = np.asarray(data)
        self.grad: Optional[np.ndarray] = None
        self.op = op
        self.name = name
        self.parents: Sequence["Tensor"] = ()
        self.backward_rule: Optional[Callable[[], None]] = None

    # --- properties used by the ops
    @property
    def shape(self):
        return self.data.shape

    @property
    def size(self):
        return self.data.size

    @property
    def is_leaf(self):
        return self.op == "leaf"

    def item(self):
        return self.data.reshape(-1)[0]

    def grad_buf(self) -> np.ndarray:
        if self.grad is None:
            self.grad = np.zeros_like(self.data)
        return self.grad

    def zero_grad(self):
        if self.grad is not None:
            self.grad[...] = 0

    def accumulate(self, g: np.ndarray):
        gb = self.grad_buf()
        gb += g.reshape(gb.shape).astype(gb.dtype, copy=False)

    # --- the tape
    @staticmethod
    def make(data, op: str, inputs: Sequence["Tensor"], rule_for: Callable[["Tensor"], Callable[[], None]]):
        t = Tensor(data, op)
        if not _no_grad[0]:
            t.parents = tuple(inputs)
            t.backward_rule = rule_for(t)
        return t

    def topological_order(self) -> List["Tensor"]:
        """Iterative depth-first search: a node is emitted after all its parents."""
        order: List[Tensor] = []
        visited = set()
        stack = [(self, False)]
        while stack:
            node, expanded = stack.pop()
            if expanded:
                order.append(node)
                continue
            if id(node) in visited:
                continue
            visited.add(id(node))
            stack.append((node, True))
            for p in node.parents:
                if id(p) not in visited:
                    stack.append((p, False))
        return order

    def backward(self):
        if self.size != 1:
            raise ValueError("backward() starts from a scalar loss")
        order = self.topological_order()
        for t in order:
            if not t.is_leaf:
                t.zero_grad()
        self.grad_buf().reshape(-1)[0] = 1
        for t in reversed(order):
            if t.backward_rule is not None:
                t.backward_rule()


# --------------------------------------------------------------------------
# Ops on tensors: the forward value and the accumulate-into-inputs rule
# --------------------------------------------------------------------------
def add(a: Tensor, b: Tensor) -> Tensor:
    def rule(o):
        def r():
            da, db = O.add_bwd(o.grad, a.shape, b.shape)
            a.accumulate(da)
            b.accumulate(db)
        return r
    return Tensor.make(O.add_fwd(a.data, b.data), "add", [a, b], rule)


def mul(a: Tensor, b: Tensor) -> Tensor:
    def rule(o):
        def r():
            da, db = O.mul_bwd(o.grad, a.data, b.data)
            a.accumulate(da)
            b.accumulate(db)
        return r
    return Tensor.make(O.mul_fwd(a.data, b.data), "mul", [a, b], rule)


def mul_assign_wrong(a: Tensor, b: Tensor) -> Tensor:
    """A deliberately wrong Mul whose rule ASSIGNS instead of adding
    ([Autograd-1, §"Why += and not ="]); used only by the negative test."""
    def rule(o):
        def r():
            da, db = O.mul_bwd(o.grad, a.data, b.data)
            a.grad_buf()[...] = da
            b.grad_buf()[...] = db
        return r
    return Tensor.make(O.mul_fwd(a.data, b.data), "mul_wrong", [a, b], rule)


def scale(a: Tensor, s: float) -> Tensor:
    def rule(o):
        return lambda: a.accumulate(O.scale_bwd(o.grad, s))
    return Tensor.make(O.scale_fwd(a.data, a.data.dtype.type(s)), "scale", [a], rule)


def sum_all(a: Tensor) -> Tensor:
    def rule(o):
        return lambda: a.accumulate(O.sum_bwd(o.grad, a.shape))
    return Tensor.make(O.sum_fwd(a.data), "sum", [a], rule)


def reshape(a: Tensor, shape) -> Tensor:
    def rule(o):
        return lambda: a.accumulate(o.grad.reshape(a.shape))
    return Tensor.make(a.data.reshape(shape).copy(), "reshape", [a], rule)


def tanh(a: Tensor) -> Tensor:
    def rule(o):
        return lambda: a.accumulate(O.tanh_bwd(o.grad, o.data))
    return Tensor.make(O.tanh_fwd(a.data), "tanh", [a], rule)


def gelu(a: Tensor) -> Tensor:
    def rule(o):
        return lambda: a.accumulate(O.gelu_bwd(o.grad, a.data))
    return Tensor.make(O.gelu_fwd(a.data), "gelu", [a], rule)


def matmul(x: Tensor, w: Tensor) -> Tensor:
    def rule(o):
        def r():
            dx, dw = O.matmul_bwd(o.grad, x.data, w.data)
            x.accumulate(dx)
            w.accumulate(dw)
        return r
    return Tensor.make(O.matmul_fwd(x.data, w.data), "matmul", [x, w], rule)


def matmul_t(x: Tensor, w: Tensor) -> Tensor:
    def rule(o):
        def r():
            dx, dw = O.matmul_t_bwd(o.grad, x.data, w.data)
            x.accumulate(dx)
            w.accumulate(dw)
        return r
    return Tensor.make(O.matmul_t_fwd(x.data, w.data), "matmul_t", [x, w], rule)


def batch_matmul(a: Tensor, b: Tensor) -> Tensor:
    def rule(o):
        def r():
            da, db = O.batch_matmul_bwd(o.grad, a.data, b.data)
            a.accumulate(da)
            b.accumulate(db)
        return r
    return Tensor.make(O.batch_matmul_fwd(a.data, b.data), "batch_matmul", [a, b], rule)


def batch_matmul_t(a: Tensor, b: Tensor) -> Tensor:
    def rule(o):
        def r():
            da, db = O.batch_matmul_t_bwd(o.grad, a.data, b.data)
            a.accumulate(da)
            b.accumulate(db)
        return r
    return Tensor.make(O.batch_matmul_t_fwd(a.data, b.data), "batch_matmul_t", [a, b], rule)


def embedding(table: Tensor, ids, batch: int) -> Tensor:
    ids = np.asarray(ids).reshape(-1).copy()

    def rule(o):
        return lambda: table.accumulate(O.embedding_bwd(o.grad, ids, table.shape))
    return Tensor.make(O.embedding_fwd(table.data, ids, batch), "embedding", [table], rule)


def layernorm(x: Tensor, gamma: Tensor, beta: Tensor, eps: float = O.LN_EPS) -> Tensor:
    y, mu, rstd = O.layernorm_fwd(x.data, gamma.data, beta.data, eps)

    def rule(o):
        def r():
            dx, dg, db = O.layernorm_bwd(o.grad, x.data, gamma.data, mu, rstd)
            x.accumulate(dx)
            gamma.accumulate(dg)
            beta.accumulate(db)
        return r
    return Tensor.make(y, "layernorm", [x, gamma, beta], rule)


def softmax_cross_entropy(logits: Tensor, targets) -> Tensor:
    targets = np.asarray(targets).reshape(-1).copy()
    loss, probs = O.softmax_ce_fwd(logits.data, targets)

    def rule(o):
        return lambda: logits.accumulate(O.softmax_ce_bwd(o.grad, probs, targets))
    return Tensor.make(loss, "softmax_ce", [logits], rule)


def causal_softmax(s: Tensor) -> Tensor:
    def rule(o):
        return lambda: s.accumulate(O.causal_softmax_bwd(o.grad, o.data))
    return Tensor.make(O.causal_softmax_fwd(s.data), "causal_softmax", [s], rule)


def narrow(x: Tensor, start: int, length: int) -> Tensor:
    def rule(o):
        return lambda: x.accumulate(O.narrow_bwd(o.grad, x.shape, start))
    return Tensor.make(O.narrow_fwd(x.data, start, length), "narrow", [x], rule)


def split_heads(x: Tensor, heads: int) -> Tensor:
    def rule(o):
        return lambda: x.accumulate(O.split_heads_bwd(o.grad))
    return Tensor.make(O.split_heads_fwd(x.data, heads), "split_heads", [x], rule)


def merge_heads(x: Tensor) -> Tensor:
    heads = x.shape[1]

    def rule(o):
        return lambda: x.accumulate(O.merge_heads_bwd(o.grad, heads))
    return Tensor.make(O.merge_heads_fwd(x.data), "merge_heads", [x], rule)
