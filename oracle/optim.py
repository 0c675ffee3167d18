"""SGD and AdamW as step-by-step updates of the parameters.

Test infrastructure only.  [Autograd-1, §"The Optimizer: from gradient to a step"]:

SGD:   w <- w - lr * g, skipping parameters that have no gradient.

AdamW (decoupled weight decay): per step t <- t + 1, bc1 = 1 - beta1^t,
bc2 = 1 - beta2^t; for every parameter that has a gradient, weight decay wd
applies only to tensors of rank >= 2 (biases and LayerNorm gains are not
decayed); per element
    m <- beta1 m + (1 - beta1) g
    v <- beta2 v + (1 - beta2) g^2
    p <- p - lr * ( (m / bc1) / (sqrt(v / bc2) + eps) + wd * p )
where the p inside the parenthesis is the value before this step.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from . import engine as E


class Optimizer:
    def __init__(self, params: Sequence[E.Tensor], lr: float):
        self.params = list(params)
        self.lr = lr

    def zero_grad(self):
        for p in self.params:
            p.zero_grad()


class SGD(Optimizer):
    def step(self):
        for p in self.params:
            if p.grad is None:
                continue
            p.data -= self.lr * p.grad


class AdamW(Optimizer):
    def __init__(self, params, lr, weight_decay=0.01, beta1=0.9, beta2=0.999, eps=1e-8):
        super().__init__(params, lr)
        self.wd, self.b1, self.b2, self.eps = weight_decay, beta1, beta2, eps
        self.m = [np.zeros_like(p.data) for p in self.params]
        self.v = [np.zeros_like(p.data) for p in self.params]
        self.t = 0

    def step(self):
        self.t += 1
        bc1 = 1 - self.b1 ** self.t
        bc2 = 1 - self.b2 ** self.t
        for k, p in enumerate(self.params):
            if p.grad is None:
                continue
            wd = self.wd if p.data.ndim >= 2 else 0.0
            g = p.grad
            self.m[k] = self.b1 * self.m[k] + (1 - self.b1) * g
            self.v[k] = self.b2 * self.v[k] + (1 - self.b2) * g * g
            mhat = self.m[k] / bc1
            vhat = self.v[k] / bc2
            p.data -= self.lr * (mhat / (np.sqrt(vhat) + self.eps) + wd * p.data)
