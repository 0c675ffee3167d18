"""KV-cached single-token inference and top-k / temperature sampling.

Test infrastructure only.  [GPT2-4, §"Generation with KV cache"]: one new token
at position pos goes through every block; each block's attention computes
qkv = c_attn(x), appends the token's key and value to that layer's cache, and
for every head takes scores_j = (q . k_j) / sqrt(hs) over all cached positions
j (no mask: the cache holds only the past), p = softmax(scores),
y_head = sum_j p_j v_j; then the output projection.  The step's logits are
MatMulT(LN_f(x), wte).

[GPT2-4, §"Temperature and Top-k"]: copy the logits, find the k-th largest
value, set every logit strictly below it to -inf (ties with it survive),
softmax with temperature (sum in double), then draw.  The draw itself is not
shown on the page; it is read here as the inverse CDF over ascending token id
with a uniform u in [0, 1) supplied by the caller.
"""
from __future__ import annotations

import math
from typing import Dict, List

import numpy as np

from . import ops as O


def _ln(x, P, name):
    y, _, _ = O.layernorm_fwd(x, P[name + ".weight"], P[name + ".bias"])
    return y


class KvCache:
    """Per layer: keys and values of every position seen so far, per sequence."""

    def __init__(self, n_layer: int):
        self.k: List[list] = [[] for _ in range(n_layer)]
        self.v: List[list] = [[] for _ in range(n_layer)]

    def length(self, layer: int) -> int:
        return len(self.k[layer])


def step(P: Dict[str, np.ndarray], tokens: np.ndarray, pos: int, cache: KvCache,
         n_layer: int, n_head: int) -> np.ndarray:
    """Batch of B sequences, one new token each at position pos -> logits [B, V]."""
    x = P["wte.weight"][tokens] + P["wpe.weight"][pos][None, :]
    B, C = x.shape
    hs = C // n_head
    for i in range(n_layer):
        pre = f"h.{i}."
        h = _ln(x, P, pre + "ln_1")
        qkv = h @ P[pre + "attn.c_attn.weight"] + P[pre + "attn.c_attn.bias"]
        cache.k[i].append(qkv[:, C:2 * C].copy())
        cache.v[i].append(qkv[:, 2 * C:].copy())
        K = np.stack(cache.k[i], axis=1)   # [B, t, C]
        V = np.stack(cache.v[i], axis=1)
        y = np.zeros((B, C))
        for hd in range(n_head):
            sl = slice(hd * hs, (hd + 1) * hs)
            for b in range(B):
                scores = K[b, :, sl] @ qkv[b, sl] / math.sqrt(hs)
                p = O.softmax_row(scores)
                y[b, sl] = p @ V[b, :, sl]
        x = x + (y @ P[pre + "attn.c_proj.weight"] + P[pre + "attn.c_proj.bias"])
        h = _ln(x, P, pre + "ln_2")
        f = O.gelu_fwd(h @ P[pre + "mlp.c_fc.weight"] + P[pre + "mlp.c_fc.bias"])
        x = x + (f @ P[pre + "mlp.c_proj.weight"] + P[pre + "mlp.c_proj.bias"])
    return _ln(x, P, "ln_f") @ P["wte.weight"].T


def top_k_temperature_probs(logits: np.ndarray, k: int, temperature: float) -> np.ndarray:
    l = np.array(logits, dtype=np.float64)
    if 0 < k < l.size:
        kth = np.sort(l)[::-1][k - 1]
        l[l < kth] = -np.inf
    return O.softmax_row(l, temperature)


def sample(probs: np.ndarray, u: float) -> int:
    """First id j (ascending) whose cumulative probability exceeds u; if rounding
    leaves none, the last id with p > 0."""
    c = np.cumsum(probs)
    j = int(np.searchsorted(c, u, side="right"))
    if j >= probs.size or probs[j] == 0:
        j = int(np.nonzero(probs > 0)[0][-1])
    return j
