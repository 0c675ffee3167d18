"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws numbers: shapes, seeds and distributions of the five
workloads.  It holds none of the method's arithmetic (no op, no gradient, no
optimizer step), so both the CPU oracle and the HIP path can take their inputs
from it without sharing any computation.

Workloads (sizes follow the GPT of "Build a language model in C# from scratch",
parts 1 and 4 -- the Tensor/Ops tables and the GPT-2 loading section):

  tiny_mlp   Linear 16->32 tanh -> 32->32 tanh -> 32->4, batch 64, fp32
  char_mlp   vocab 64, context 8, embedding 24 (concatenated to 192) ->
             Linear 192->256 tanh -> 256->64, batch 256
  tiny_gpt   vocab 64, n_embd 128, 4 heads, 2 pre-LN blocks, context 64, batch 32
  gpt2       vocab 50257, n_embd 768, 12 heads, 12 layers, context 1024, batch 8
  gpt2_infer same weights as gpt2; batch 16, prompt 768, 256 sampled steps

All draws use numpy's PCG64 generator; the seed of workload n (1..5) is 2026+n.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Tuple

import numpy as np

SEED_BASE = 2026


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ----------------------------------------------------------------------------
# GPT shapes
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class GptShape:
    vocab: int
    n_positions: int
    n_layer: int
    n_head: int
    n_embd: int

    @property
    def head_size(self) -> int:
        return self.n_embd // self.n_head


TINY_GPT = GptShape(vocab=64, n_positions=64, n_layer=2, n_head=4, n_embd=128)
GPT2_124M = GptShape(vocab=50257, n_positions=1024, n_layer=12, n_head=12, n_embd=768)


def gpt_param_shapes(s: GptShape) -> List[Tuple[str, Tuple[int, ...]]]:
    """Parameter names and shapes in GPT-2's naming (weights stored [in, out])."""
    C = s.n_embd
    out = [("wte.weight", (s.vocab, C)), ("wpe.weight", (s.n_positions, C))]
    for i in range(s.n_layer):
        p = f"h.{i}."
        out += [
            (p + "ln_1.weight", (C,)), (p + "ln_1.bias", (C,)),
            (p + "attn.c_attn.weight", (C, 3 * C)), (p + "attn.c_attn.bias", (3 * C,)),
            (p + "attn.c_proj.weight", (C, C)), (p + "attn.c_proj.bias", (C,)),
            (p + "ln_2.weight", (C,)), (p + "ln_2.bias", (C,)),
            (p + "mlp.c_fc.weight", (C, 4 * C)), (p + "mlp.c_fc.bias", (4 * C,)),
            (p + "mlp.c_proj.weight", (4 * C, C)), (p + "mlp.c_proj.bias", (C,)),
        ]
    out += [("ln_f.weight", (C,)), ("ln_f.bias", (C,))]
    return out


def gpt_params(s: GptShape, seed: int, std: float = 0.02) -> Dict[str, np.ndarray]:
    """Random init: matrices N(0, std^2), biases 0, LayerNorm gains 1 and shifts 0."""
    rng = rng_for(seed)
    params: Dict[str, np.ndarray] = {}
    for name, shape in gpt_param_shapes(s):
        if len(shape) == 2:
            a = rng.standard_normal(shape, dtype=np.float32)
            a *= np.float32(std)
        elif ".ln_" in name or name.startswith("ln_f"):
            a = np.ones(shape, np.float32) if name.endswith("weight") else np.zeros(shape, np.float32)
        else:
            a = np.zeros(shape, np.float32)
        params[name] = a
    return params


def token_batch(seed: int, batch: int, length: int, vocab: int) -> np.ndarray:
    """ids [batch, length+1] uniform in [0, vocab): inputs are [:, :-1], targets [:, 1:]."""
    return rng_for(seed).integers(0, vocab, size=(batch, length + 1), dtype=np.int64).astype(np.int32)


# ----------------------------------------------------------------------------
# The five workloads
# ----------------------------------------------------------------------------
def tiny_mlp(seed: int = SEED_BASE + 1):
    """Tiny MLP: X ~ N(0,1) [64,16], labels uniform {0..3}, W ~ N(0, 1/fan_in), b = 0."""
    rng = rng_for(seed)
    sizes = [16, 32, 32, 4]
    params = {}
    for i in range(3):
        fan_in, fan_out = sizes[i], sizes[i + 1]
        params[f"w{i + 1}"] = (rng.standard_normal((fan_in, fan_out)) / np.sqrt(fan_in)).astype(np.float32)
        params[f"b{i + 1}"] = np.zeros((fan_out,), np.float32)
    x = rng.standard_normal((64, 16)).astype(np.float32)
    y = rng.integers(0, 4, size=(64,), dtype=np.int64).astype(np.int32)
    return params, x, y


def char_mlp(seed: int = SEED_BASE + 2):
    """Char-level MLP LM: table N(0,1) [64,24]; Linear weights N(0, 1/fan_in); biases 0."""
    rng = rng_for(seed)
    params = {
        "emb": rng.standard_normal((64, 24)).astype(np.float32),
        "w1": (rng.standard_normal((192, 256)) / np.sqrt(192)).astype(np.float32),
        "b1": np.zeros((256,), np.float32),
        "w2": (rng.standard_normal((256, 64)) / np.sqrt(256)).astype(np.float32),
        "b2": np.zeros((64,), np.float32),
    }
    return params


def char_mlp_batch(step: int, seed: int = SEED_BASE + 2, batch: int = 256):
    """A fresh [256, 9] id draw per step: context ids [:, :8], target [:, 8]."""
    ids = rng_for(seed * 1000 + step).integers(0, 64, size=(batch, 9), dtype=np.int64).astype(np.int32)
    return ids[:, :8].copy(), ids[:, 8].copy()


def tiny_gpt(seed: int = SEED_BASE + 3, batch: int = 32):
    s = TINY_GPT
    params = gpt_params(s, seed)
    ids = token_batch(seed + 100, batch, s.n_positions, s.vocab)
    return s, params, ids


def gpt2(seed: int = SEED_BASE + 4, batch: int = 8, seq: int = 1024):
    s = GPT2_124M
    params = gpt_params(s, seed)
    ids = token_batch(seed + 100, batch, seq, s.vocab)
    return s, params, ids


def gpt2_infer(seed: int = SEED_BASE + 5, batch: int = 16, prompt: int = 768, steps: int = 256):
    """Same shapes as gpt2; prompts [16, 768] uniform ids; sampling uniforms u[16, 256] (float64)."""
    s = GPT2_124M
    params = gpt_params(s, SEED_BASE + 4)
    rng = rng_for(seed)
    prompts = rng.integers(0, s.vocab, size=(batch, prompt), dtype=np.int64).astype(np.int32)
    uniforms = rng.random((batch, steps))
    return s, params, prompts, uniforms


def random_array(seed: int, shape, scale: float = 1.0, dtype=np.float32) -> np.ndarray:
    """Generic N(0, scale^2) array for per-op tests."""
    return (rng_for(seed).standard_normal(shape) * scale).astype(dtype)


def random_ids(seed: int, shape, high: int) -> np.ndarray:
    return rng_for(seed).integers(0, high, size=shape, dtype=np.int64).astype(np.int32)
