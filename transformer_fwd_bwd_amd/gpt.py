"""The workloads composed from libtfb ops: tiny MLP, char-level MLP and the GPT.

Composition follows the pages ([Autograd-1, "Training loop": Linear = MatMul +
bias Add, Tanh, SoftmaxCrossEntropy; GPT2-4, "Loading the weights" and
"Generation with KV cache": token + position embedding, pre-LN blocks with a
fused c_attn [C, 3C], MLP C -> 4C -> C with GELU, ln_f, the LM head tied to
wte).  Linear is the fused MatMul+bias op (with the residual Add folded in where a
projection feeds the residual stream) and the attention core is the single
tfb_causal_attention op; each computes exactly the pages' op sequence.
"""
from __future__ import annotations

from typing import Dict, List, Sequence

import numpy as np

from . import (AdamW, Context, KvCache, Tensor, add, causal_attention, embedding, gelu, layernorm, linear,
               matmul_t, mlp_residual_layernorm, narrow, reshape, sample_topk, softmax_cross_entropy, tanh)


def upload_params(ctx: Context, params: Dict[str, np.ndarray]) -> Dict[str, Tensor]:
    return {k: ctx.tensor(v.shape, v, param=True, name=k) for k, v in params.items()}


class Gpt:
    def __init__(self, ctx: Context, n_layer: int, n_head: int, params: Dict[str, np.ndarray]):
        self.ctx = ctx
        self.n_layer, self.n_head = n_layer, n_head
        self.P = upload_params(ctx, params)
        self.names = list(params.keys())
        self._pos = {}

    @property
    def param_list(self) -> List[Tensor]:
        return [self.P[k] for k in self.names]

    def positions(self, T: int):
        if T not in self._pos:
            import torch
            self._pos[T] = torch.arange(T, dtype=torch.int32, device=f"cuda:{self.ctx.device}")
        return self._pos[T]

    def hidden(self, ids) -> Tensor:
        """ids: [B, T] int32 (numpy or a device torch tensor) -> the last block's output [B, T, C]."""
        P = self.P
        B, T = ids.shape
        C = P["wte.weight"].shape[1]
        if T > P["wpe.weight"].shape[0]:
            raise ValueError(f"{T} positions exceed the {P['wpe.weight'].shape[0]} position embeddings")
        tok = embedding(P["wte.weight"], ids, B)                          # [B, T, C]
        pos = reshape(embedding(P["wpe.weight"], self.positions(T), 1), (T, C))
        x = add(tok, pos)
        # Outputs whose only readers are contractions, the fused attention, the GELU or
        # the cross-entropy are kept as bf16 copies alone in the bf16 variant (the
        # LayerNorms', qkv, the attention's, the MLP's first product, the GELU's, the logits)
        for i in range(self.n_layer):
            p = f"h.{i}."
            h = layernorm(x, P[p + "ln_1.weight"], P[p + "ln_1.bias"], bf16_only=True)
            qkv = linear(h, P[p + "attn.c_attn.weight"], P[p + "attn.c_attn.bias"], bf16_only=True)
            a = causal_attention(qkv, self.n_head, bf16_only=True)
            x = linear(a, P[p + "attn.c_proj.weight"], P[p + "attn.c_proj.bias"], residual=x)
            h = layernorm(x, P[p + "ln_2.weight"], P[p + "ln_2.bias"], bf16_only=True)
            f = gelu(linear(h, P[p + "mlp.c_fc.weight"], P[p + "mlp.c_fc.bias"], bf16_only=True), bf16_only=True)
            x = linear(f, P[p + "mlp.c_proj.weight"], P[p + "mlp.c_proj.bias"], residual=x)
        return x

    def logits(self, ids) -> Tensor:
        """ids: [B, T] int32 (numpy or a device torch tensor) -> logits [B, T, V]."""
        P = self.P
        xf = layernorm(self.hidden(ids), P["ln_f.weight"], P["ln_f.bias"], bf16_only=True)
        return matmul_t(xf, P["wte.weight"], bf16_only=True)   # read by the fused cross-entropy

    def loss(self, inputs, targets):
        """(mean cross-entropy, logits).  In the bf16 variant the logits' gradient exists
        only as the bf16 copy the LM head's backward reads (it is not kept in fp32)."""
        logits = self.logits(inputs)
        return softmax_cross_entropy(logits, targets, bf16_grad_only=True), logits

    # ------------------------------------------------------------------ KV-cached inference
    # [GPT2-4, "Generation with KV cache"]: the prompt's keys and values are
    # computed once (here in one batched pass instead of token by token -- the
    # same arithmetic), then each new token runs through every block alone,
    # attending over the cached past.

    def prefill(self, ids, kv: KvCache):
        """Run positions 0..P-1 of ids [B, P] through the blocks, storing every layer's keys/values."""
        P = self.P
        B, T = ids.shape
        C = P["wte.weight"].shape[1]
        x = add(embedding(P["wte.weight"], ids, B), reshape(embedding(P["wpe.weight"], self.positions(T), 1), (T, C)))
        for i in range(self.n_layer):
            p = f"h.{i}."
            h = layernorm(x, P[p + "ln_1.weight"], P[p + "ln_1.bias"])
            qkv = linear(h, P[p + "attn.c_attn.weight"], P[p + "attn.c_attn.bias"])
            kv.store(i, qkv, 0)
            if i == self.n_layer - 1:
                break   # the last block's output is not needed: the next token comes from a decode step
            a = causal_attention(qkv, self.n_head)
            x = linear(a, P[p + "attn.c_proj.weight"], P[p + "attn.c_proj.bias"], residual=x)
            h = layernorm(x, P[p + "ln_2.weight"], P[p + "ln_2.bias"])
            f = gelu(linear(h, P[p + "mlp.c_fc.weight"], P[p + "mlp.c_fc.bias"]))
            x = linear(f, P[p + "mlp.c_proj.weight"], P[p + "mlp.c_proj.bias"], residual=x)

    def decode_step(self, tokens, pos: int, kv: KvCache, tmax: int) -> Tensor:
        """One token per sequence (tokens: [B] int32) at position pos -> logits [B, 1, V]."""
        P = self.P
        B = tokens.shape[0]
        C = P["wte.weight"].shape[1]
        x = add(embedding(P["wte.weight"], tokens, B),
                reshape(embedding(P["wpe.weight"], self.positions(tmax)[pos:pos + 1], 1), (1, C)))
        # the same ops in fewer passes: each LayerNorm is folded into the chunk sum of
        # the residual projection before it, the c_attn product's chunk sum into the
        # cached attention's loads, the attention's merge of its position blocks into
        # the projection's loads, and the MLP's hidden activation (c_fc and GELU) into
        # the MLP projection's loads
        h = layernorm(x, P["h.0.ln_1.weight"], P["h.0.ln_1.bias"], bf16_only=True)
        for i in range(self.n_layer):
            p = f"h.{i}."
            x, h = kv.attention_block(i, h, P[p + "attn.c_attn.weight"], P[p + "attn.c_attn.bias"], pos,
                                      self.n_head, P[p + "attn.c_proj.weight"], P[p + "attn.c_proj.bias"], x,
                                      P[p + "ln_2.weight"], P[p + "ln_2.bias"], bf16_only=True)
            ln = f"h.{i + 1}.ln_1" if i + 1 < self.n_layer else "ln_f"
            x, h = mlp_residual_layernorm(h, P[p + "mlp.c_fc.weight"], P[p + "mlp.c_fc.bias"],
                                          P[p + "mlp.c_proj.weight"], P[p + "mlp.c_proj.bias"], x,
                                          P[ln + ".weight"], P[ln + ".bias"], bf16_only=True)
        return matmul_t(h, P["wte.weight"])

    def generate(self, prompts, steps: int, uniforms, k: int, temperature: float, on_step=None):
        """[GPT2-4, "Temperature and Top-k"]: prompts [B, P] (device int32), uniforms [B, steps]
        (device float64).  Returns the sampled ids [B, steps] (device int32).  on_step(i, logits,
        token) sees every step's logits before the tape is reset."""
        import torch
        ctx = self.ctx
        B, Pn = prompts.shape
        tmax = Pn + steps - 1
        C = self.P["wte.weight"].shape[1]
        if tmax > self.P["wpe.weight"].shape[0]:
            raise ValueError(f"{tmax} positions exceed the {self.P['wpe.weight'].shape[0]} position embeddings")
        kv = KvCache(ctx, self.n_layer, B, max(tmax, 1), C)
        out = torch.empty((steps, B), dtype=torch.int32, device=f"cuda:{ctx.device}")
        u = uniforms.t().contiguous()
        ctx.set_grad_enabled(False)
        try:
            if Pn > 1:
                self.prefill(prompts[:, :-1].contiguous(), kv)
                ctx.tape_reset()
            tok = prompts[:, -1].contiguous()
            for i in range(steps):
                logits = self.decode_step(tok, Pn - 1 + i, kv, tmax)
                sample_topk(logits, k, temperature, u[i], out=out[i])
                if on_step is not None:
                    on_step(i, logits, out[i])
                ctx.tape_reset()
                tok = out[i]
        finally:
            ctx.set_grad_enabled(True)
            kv.close()
        return out.t().contiguous()

    def generate_uncached(self, prompts, steps: int, uniforms, k: int, temperature: float, on_step=None):
        """[GPT2-4, "Generation with KV cache", the variant without a cache]: every new token runs
        the whole forward over the sequence so far and samples from its last position.  Same
        arguments and result as generate(); only the last position goes through ln_f and the
        LM head."""
        import torch
        ctx = self.ctx
        P = self.P
        B, Pn = prompts.shape
        C = P["wte.weight"].shape[1]
        if Pn < 1:
            raise ValueError("an empty prompt has no last position")
        if Pn + steps - 1 > P["wpe.weight"].shape[0]:
            raise ValueError(f"{Pn + steps - 1} positions exceed the {P['wpe.weight'].shape[0]} position embeddings")
        out = torch.empty((steps, B), dtype=torch.int32, device=f"cuda:{ctx.device}")
        u = uniforms.t().contiguous()
        seq = prompts.contiguous()
        ctx.set_grad_enabled(False)
        try:
            for i in range(steps):
                T = seq.shape[1]
                x = reshape(self.hidden(seq), (B, T * C))
                last = narrow(x, (T - 1) * C, C)                              # [B, C]
                logits = matmul_t(layernorm(last, P["ln_f.weight"], P["ln_f.bias"]), P["wte.weight"])
                sample_topk(logits, k, temperature, u[i], out=out[i])
                if on_step is not None:
                    on_step(i, logits, out[i])
                ctx.tape_reset()
                if i + 1 < steps:
                    seq = torch.cat([seq, out[i][:, None]], dim=1)
        finally:
            ctx.set_grad_enabled(True)
        return out.t().contiguous()


def split_ids(ids_full):
    """[B, T+1] -> inputs [B, T], targets [B*T] (works for numpy and torch)."""
    inputs = ids_full[:, :-1]
    targets = ids_full[:, 1:]
    if hasattr(inputs, "contiguous"):
        return inputs.contiguous(), targets.contiguous().reshape(-1)
    return np.ascontiguousarray(inputs), np.ascontiguousarray(targets).reshape(-1)


def train_step(model: Gpt, opt: AdamW, inputs, targets, read_loss: bool = True):
    """One fwd + backward + AdamW step; returns the loss (or None)."""
    ctx = model.ctx
    loss, _ = model.loss(inputs, targets)
    opt.zero_grad()
    ctx.backward(loss)
    opt.step()
    val = loss.item() if read_loss else None
    ctx.tape_reset()
    return val


class TinyMlp:
    """Linear 16->32 tanh -> 32->32 tanh -> 32->4."""

    def __init__(self, ctx: Context, params: Dict[str, np.ndarray]):
        self.ctx = ctx
        self.P = upload_params(ctx, params)
        self.names = list(params.keys())

    @property
    def param_list(self):
        return [self.P[k] for k in self.names]

    def loss(self, x: Tensor, y):
        P = self.P
        h = tanh(linear(x, P["w1"], P["b1"]))
        h = tanh(linear(h, P["w2"], P["b2"]))
        logits = linear(h, P["w3"], P["b3"])
        return softmax_cross_entropy(logits, y), logits


class CharMlp:
    """Embedding 64x24 of 8 context ids, concatenated to 192 -> 256 tanh -> 64."""

    def __init__(self, ctx: Context, params: Dict[str, np.ndarray]):
        self.ctx = ctx
        self.P = upload_params(ctx, params)
        self.names = list(params.keys())

    @property
    def param_list(self):
        return [self.P[k] for k in self.names]

    def loss(self, ctx_ids, target):
        P = self.P
        B, K = ctx_ids.shape
        emb = embedding(P["emb"], ctx_ids, B)
        x = reshape(emb, (B, K * P["emb"].shape[1]))
        h = tanh(linear(x, P["w1"], P["b1"]))
        logits = linear(h, P["w2"], P["b2"])
        return softmax_cross_entropy(logits, target), logits
