"""The workloads composed from the oracle's ops.

Test infrastructure only.

* tiny MLP and char-level MLP: Linear = MatMul followed by a broadcast Add of the
  bias, Tanh between layers, SoftmaxCrossEntropy at the end ([Autograd-1,
  §"Training loop": the same composition for the circle classifier]).
* GPT (pre-LN): h0 = Embedding(wte, ids) + Embedding(wpe, 0..T-1); per block
  x = x + Attn(LN1(x)), x = x + MLP(LN2(x)); logits = MatMulT(LN_f(x), wte)
  ([GPT2-4, §"Loading the weights": Linear weights stored [in, out], q/k/v fused
  in c_attn [C, 3C], MLP C -> 4C -> C, the LM head tied to wte; §"Generation
  with KV cache": the embedding sum and the LM head]).
* attention: qkv = x W + b; q, k, v = Narrow thirds; heads are contiguous
  slices of hs = C/H columns; S = (q k^T) * 1/sqrt(hs); P = CausalSoftmax(S);
  O = P v; MergeHeads; output projection ([Autograd-1, table of ops;
  GPT2-4, §"Generation with KV cache"]).
"""
from __future__ import annotations

import math
from typing import Dict, List, Tuple

import numpy as np

from . import engine as E


def as_tensors(params: Dict[str, np.ndarray], dtype=np.float64) -> Dict[str, E.Tensor]:
    return {k: E.Tensor(np.array(v, dtype=dtype), name=k) for k, v in params.items()}


def linear(x: E.Tensor, w: E.Tensor, b: E.Tensor) -> E.Tensor:
    return E.add(E.matmul(x, w), b)


# --------------------------------------------------------------------------
def tiny_mlp_loss(P: Dict[str, E.Tensor], x: np.ndarray, y: np.ndarray):
    xt = E.Tensor(np.asarray(x, dtype=P["w1"].data.dtype))
    h = E.tanh(linear(xt, P["w1"], P["b1"]))
    h = E.tanh(linear(h, P["w2"], P["b2"]))
    logits = linear(h, P["w3"], P["b3"])
    return E.softmax_cross_entropy(logits, y), logits


def char_mlp_loss(P: Dict[str, E.Tensor], ctx_ids: np.ndarray, target: np.ndarray):
    B, K = ctx_ids.shape
    emb = E.embedding(P["emb"], ctx_ids.reshape(-1), B)          # [B, 8, 24]
    x = E.reshape(emb, (B, K * P["emb"].shape[1]))                # [B, 192]
    h = E.tanh(linear(x, P["w1"], P["b1"]))
    logits = linear(h, P["w2"], P["b2"])
    return E.softmax_cross_entropy(logits, target), logits


# --------------------------------------------------------------------------
def attention(x: E.Tensor, P: Dict[str, E.Tensor], pre: str, n_head: int) -> E.Tensor:
    C = x.shape[-1]
    hs = C // n_head
    qkv = linear(x, P[pre + "attn.c_attn.weight"], P[pre + "attn.c_attn.bias"])
    q = E.split_heads(E.narrow(qkv, 0, C), n_head)
    k = E.split_heads(E.narrow(qkv, C, C), n_head)
    v = E.split_heads(E.narrow(qkv, 2 * C, C), n_head)
    B, H, T, _ = q.shape
    q3 = E.reshape(q, (B * H, T, hs))
    k3 = E.reshape(k, (B * H, T, hs))
    v3 = E.reshape(v, (B * H, T, hs))
    s = E.scale(E.batch_matmul_t(q3, k3), 1.0 / math.sqrt(hs))
    p = E.causal_softmax(s)
    o = E.reshape(E.batch_matmul(p, v3), (B, H, T, hs))
    y = E.merge_heads(o)
    return linear(y, P[pre + "attn.c_proj.weight"], P[pre + "attn.c_proj.bias"])


def mlp(x: E.Tensor, P: Dict[str, E.Tensor], pre: str) -> E.Tensor:
    h = E.gelu(linear(x, P[pre + "mlp.c_fc.weight"], P[pre + "mlp.c_fc.bias"]))
    return linear(h, P[pre + "mlp.c_proj.weight"], P[pre + "mlp.c_proj.bias"])


def gpt_logits(P: Dict[str, E.Tensor], ids: np.ndarray, n_layer: int, n_head: int) -> E.Tensor:
    B, T = ids.shape
    tok = E.embedding(P["wte.weight"], ids.reshape(-1), B)                 # [B, T, C]
    pos = E.embedding(P["wpe.weight"], np.arange(T), 1)                    # [1, T, C]
    x = E.add(tok, E.reshape(pos, (T, pos.shape[-1])))
    for i in range(n_layer):
        pre = f"h.{i}."
        x = E.add(x, attention(E.layernorm(x, P[pre + "ln_1.weight"], P[pre + "ln_1.bias"]), P, pre, n_head))
        x = E.add(x, mlp(E.layernorm(x, P[pre + "ln_2.weight"], P[pre + "ln_2.bias"]), P, pre))
    xf = E.layernorm(x, P["ln_f.weight"], P["ln_f.bias"])
    return E.matmul_t(xf, P["wte.weight"])


def gpt_loss(P, ids_full: np.ndarray, n_layer: int, n_head: int):
    """ids_full [B, T+1]: inputs [:, :T], targets [:, 1:]."""
    inputs, targets = ids_full[:, :-1], ids_full[:, 1:]
    logits = gpt_logits(P, inputs, n_layer, n_head)
    return E.softmax_cross_entropy(logits, targets.reshape(-1)), logits


def param_count(shapes: List[Tuple[str, Tuple[int, ...]]]) -> int:
    return int(sum(np.prod(s) for _, s in shapes))
