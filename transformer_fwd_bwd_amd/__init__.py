"""Python binding of libtfb, the MI355X (gfx950) tensor-autograd library.

Argument marshalling only: every op runs in the library's HIP kernels.  PyTorch
supplies the device arena (one uint8 tensor) and the HIP stream; numpy arrays
cross the boundary through tfb_tensor_write / tfb_tensor_read.  The library must
be built (see build.py); importing ops without it raises immediately -- there
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtfb.so")

FP32 = 0
BF16_MFMA = 1
_PREC = {"fp32": FP32, "bf16": BF16_MFMA, FP32: FP32, BF16_MFMA: BF16_MFMA}

_lib = None

# kernel families timed by Context.profile_* (TFB_PROF_* in tfb.h): name -> (id, unit of work)
PROF_KINDS = {"gemm": 0, "attn_fwd": 1, "attn_bwd": 2, "ce": 3, "adamw": 4, "ln_fwd": 5, "ln_bwd": 6, "gelu_fwd": 7,
              "gelu_bwd": 8, "gemv": 9, "kv_attend": 10, "sample": 11}
PROF_UNIT = {"gemm": "flop", "attn_fwd": "flop", "attn_bwd": "flop"}  # the others: bytes

c_int, c_int32, c_int64, c_float = ctypes.c_int, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
c_void_p, c_size_t = ctypes.c_void_p, ctypes.c_size_t
P = ctypes.POINTER

# name -> argtypes (every function returns int)
SIGNATURES = {
    "tfb_init": [P(c_void_p), c_int, c_void_p, c_void_p, c_size_t, c_int],
    "tfb_destroy": [c_void_p],
    "tfb_set_precision": [c_void_p, c_int],
    "tfb_set_grad_enabled": [c_void_p, c_int],
    "tfb_sync": [c_void_p],
    "tfb_arena_usage": [c_void_p, P(c_size_t), P(c_size_t)],
    "tfb_tensor_create": [c_void_p, P(c_int64), c_int, c_void_p, c_int, ctypes.c_char_p, P(c_int32)],
    "tfb_tensor_name": [c_void_p, c_int32, ctypes.c_char_p, c_size_t],
    "tfb_tensor_info": [c_void_p, c_int32, P(c_int64), P(c_int), P(c_void_p), P(c_void_p)],
    "tfb_tensor_write": [c_void_p, c_int32, c_void_p, c_int64],
    "tfb_tensor_read": [c_void_p, c_int32, c_int, c_void_p, c_int64],
    "tfb_tensor_release": [c_void_p, c_int32],
    "tfb_add": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_mul": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_scale": [c_void_p, c_int32, c_float, P(c_int32)],
    "tfb_sum": [c_void_p, c_int32, P(c_int32)],
    "tfb_reshape": [c_void_p, c_int32, P(c_int64), c_int, P(c_int32)],
    "tfb_tanh": [c_void_p, c_int32, P(c_int32)],
    "tfb_gelu": [c_void_p, c_int32, P(c_int32)],
    "tfb_matmul": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_matmul_t": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_matmul_t_ex": [c_void_p, c_int32, c_int32, c_int32, P(c_int32)],
    "tfb_linear": [c_void_p, c_int32, c_int32, c_int32, P(c_int32)],
    "tfb_linear_ex": [c_void_p, c_int32, c_int32, c_int32, c_int32, P(c_int32)],
    "tfb_layernorm_ex": [c_void_p, c_int32, c_int32, c_int32, c_float, c_int32, P(c_int32)],
    "tfb_gelu_ex": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_linear_residual": [c_void_p, c_int32, c_int32, c_int32, c_int32, P(c_int32)],
    "tfb_layernorm": [c_void_p, c_int32, c_int32, c_int32, c_float, P(c_int32)],
    "tfb_linear_gelu": [c_void_p, c_int32, c_int32, c_int32, c_int32, P(c_int32)],
    "tfb_mlp_residual_layernorm": [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                   c_float, c_int32, P(c_int32), P(c_int32)],
    "tfb_kv_attend_linear": [c_void_p, c_void_p, c_int, c_int32, c_int32, c_int32, c_int, c_int, P(c_int32)],
    "tfb_kv_attention_block": [c_void_p, c_void_p, c_int, c_int32, c_int32, c_int32, c_int, c_int, c_int32, c_int32,
                               c_int32, c_int32, c_int32, c_float, c_int32, P(c_int32), P(c_int32)],
    "tfb_linear_residual_layernorm": [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_float,
                                      c_int32, P(c_int32), P(c_int32)],
    "tfb_embedding": [c_void_p, c_int32, c_void_p, c_int64, c_int64, P(c_int32)],
    "tfb_narrow": [c_void_p, c_int32, c_int64, c_int64, P(c_int32)],
    "tfb_split_heads": [c_void_p, c_int32, c_int, P(c_int32)],
    "tfb_merge_heads": [c_void_p, c_int32, P(c_int32)],
    "tfb_batch_matmul": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_batch_matmul_t": [c_void_p, c_int32, c_int32, P(c_int32)],
    "tfb_causal_softmax": [c_void_p, c_int32, P(c_int32)],
    "tfb_causal_attention": [c_void_p, c_int32, c_int, P(c_int32)],
    "tfb_causal_attention_ex": [c_void_p, c_int32, c_int, c_int32, P(c_int32)],
    "tfb_softmax_cross_entropy": [c_void_p, c_int32, c_void_p, c_int64, P(c_int32)],
    "tfb_softmax_cross_entropy_ex": [c_void_p, c_int32, c_void_p, c_int64, c_int32, P(c_int32)],
    "tfb_softmax_cross_entropy_noalloc": [c_void_p, c_int64, c_void_p, c_int64, c_int64, c_void_p, c_void_p],
    "tfb_backward": [c_void_p, c_int32],
    "tfb_zero_grad": [c_void_p, P(c_int32), c_int],
    "tfb_tape_reset": [c_void_p],
    "tfb_adamw_create": [c_void_p, P(c_int32), c_int, c_float, c_float, c_float, c_float, c_float, P(c_void_p)],
    "tfb_adamw_step": [c_void_p],
    "tfb_adamw_set_lr": [c_void_p, c_float],
    "tfb_adamw_moments": [c_void_p, c_int, c_void_p, c_void_p, c_int64],
    "tfb_adamw_destroy": [c_void_p],
    "tfb_sgd_step": [c_void_p, P(c_int32), c_int, c_float],
    "tfb_kv_create": [c_void_p, c_int, c_int, c_int, c_int, P(c_void_p)],
    "tfb_kv_destroy": [c_void_p],
    "tfb_kv_store": [c_void_p, c_void_p, c_int, c_int32, c_int],
    "tfb_kv_attend": [c_void_p, c_void_p, c_int, c_int32, c_int, c_int, P(c_int32)],
    "tfb_sample_topk": [c_void_p, c_int32, c_int, c_float, c_void_p, c_void_p],
    "tfb_profile_begin": [c_void_p],
    "tfb_profile_end": [c_void_p, P(ctypes.c_double), P(ctypes.c_double), P(c_int)],
    "tfb_profile_kind": [c_void_p, c_int, P(ctypes.c_double), P(ctypes.c_double), P(c_int)],
}


class TfbError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"tfb error {code}: {msg}")
        self.code = code


def load_library(path: str = LIB_PATH):
    """Load libtfb.so and declare its signatures (no GPU is touched)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with transformer_fwd_bwd_amd.build.build()")
    lib = ctypes.CDLL(path)
    for name, argtypes in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = c_int
    for name, argtypes in _EXTRA_SIGNATURES.items():
        if hasattr(lib, name):
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = c_int
    lib.tfb_last_error.argtypes = []
    lib.tfb_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


_EXTRA_SIGNATURES: dict = {}


def _check(code: int):
    if code != 0:
        raise TfbError(code, _lib.tfb_last_error().decode())


def _i64s(seq):
    return (c_int64 * len(seq))(*seq)


class Tensor:
    """A handle owned by a Context (valid until released or, for op outputs, tape_reset)."""

    __slots__ = ("ctx", "h")

    def __init__(self, ctx: "Context", h: int):
        self.ctx, self.h = ctx, h

    @property
    def shape(self):
        shp = (c_int64 * 6)()
        nd = c_int()
        _check(_lib.tfb_tensor_info(self.ctx.ptr, self.h, shp, ctypes.byref(nd), None, None))
        return tuple(shp[i] for i in range(nd.value))

    @property
    def size(self):
        return int(np.prod(self.shape))

    def data_ptr(self) -> int:
        p = c_void_p()
        _check(_lib.tfb_tensor_info(self.ctx.ptr, self.h, None, None, ctypes.byref(p), None))
        return p.value or 0

    @property
    def name(self) -> str:
        buf = ctypes.create_string_buffer(128)
        _check(_lib.tfb_tensor_name(self.ctx.ptr, self.h, buf, 128))
        return buf.value.decode()

    def numpy(self) -> np.ndarray:
        out = np.empty(self.shape, np.float32)
        _check(_lib.tfb_tensor_read(self.ctx.ptr, self.h, 0, out.ctypes.data, out.size))
        return out

    def grad(self) -> np.ndarray:
        out = np.empty(self.shape, np.float32)
        _check(_lib.tfb_tensor_read(self.ctx.ptr, self.h, 1, out.ctypes.data, out.size))
        return out

    def write(self, arr) -> "Tensor":
        a = np.ascontiguousarray(arr, dtype=np.float32)
        _check(_lib.tfb_tensor_write(self.ctx.ptr, self.h, a.ctypes.data, a.size))
        return self

    def release(self):
        _check(_lib.tfb_tensor_release(self.ctx.ptr, self.h))

    def item(self) -> float:
        return float(self.numpy().reshape(-1)[0])


class Context:
    """One library context: a device arena (a torch uint8 tensor), torch's current
    HIP stream on that device, and the tape."""

    def __init__(self, arena_bytes: int = 1 << 30, precision="fp32", device: int = 0, stream=None):
        import torch
        load_library()
        self.device = device
        self.arena = torch.empty(int(arena_bytes), dtype=torch.uint8, device=f"cuda:{device}")
        self.stream = stream if stream is not None else torch.cuda.current_stream(device)
        ptr = c_void_p()
        _check(_lib.tfb_init(ctypes.byref(ptr), device, c_void_p(self.stream.cuda_stream),
                             c_void_p(self.arena.data_ptr()), int(arena_bytes), _PREC[precision]))
        self.ptr = ptr
        self._keep = []   # device id/target buffers kept alive until the next tape reset

    def close(self):
        if getattr(self, "ptr", None):
            _check(_lib.tfb_destroy(self.ptr))
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ----------------------------------------------------------------- state
    def set_precision(self, precision):
        _check(_lib.tfb_set_precision(self.ptr, _PREC[precision]))

    def set_grad_enabled(self, enabled: bool):
        _check(_lib.tfb_set_grad_enabled(self.ptr, int(bool(enabled))))

    def sync(self):
        _check(_lib.tfb_sync(self.ptr))

    def arena_usage(self):
        a, b = c_size_t(), c_size_t()
        _check(_lib.tfb_arena_usage(self.ptr, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def tensor(self, shape, data=None, param: bool = False, dev_ptr: Optional[int] = None, name: str = "") -> Tensor:
        shape = tuple(int(s) for s in shape)
        h = c_int32()
        _check(_lib.tfb_tensor_create(self.ptr, _i64s(shape), len(shape), c_void_p(dev_ptr) if dev_ptr else None,
                                      int(param), name.encode() if name else None, ctypes.byref(h)))
        t = Tensor(self, h.value)
        if data is not None:
            t.write(np.asarray(data, np.float32).reshape(shape))
        return t

    def device_ints(self, arr):
        """An int32 device buffer (a torch tensor) holding arr; kept alive until tape_reset."""
        import torch
        if isinstance(arr, torch.Tensor):
            t = arr.to(device=f"cuda:{self.device}", dtype=torch.int32).contiguous()
        else:
            t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32).reshape(-1)).to(f"cuda:{self.device}")
        self._keep.append(t)
        return t

    # ----------------------------------------------------------------- autograd
    def backward(self, loss: Tensor):
        _check(_lib.tfb_backward(self.ptr, loss.h))

    def zero_grad(self, params: Sequence[Tensor]):
        hs = (c_int32 * len(params))(*[p.h for p in params])
        _check(_lib.tfb_zero_grad(self.ptr, hs, len(params)))

    def profile_begin(self):
        _check(_lib.tfb_profile_begin(self.ptr))

    def profile_end(self):
        """(contraction kernel ms, algorithmic flops, launches) since profile_begin."""
        ms, fl, n = ctypes.c_double(), ctypes.c_double(), c_int()
        _check(_lib.tfb_profile_end(self.ptr, ctypes.byref(ms), ctypes.byref(fl), ctypes.byref(n)))
        return ms.value, fl.value, n.value

    def profile_kind(self, kind: int):
        """(ms, algorithmic work, launches) of one kernel family (PROF_*) after profile_end."""
        ms, w, n = ctypes.c_double(), ctypes.c_double(), c_int()
        _check(_lib.tfb_profile_kind(self.ptr, int(kind), ctypes.byref(ms), ctypes.byref(w), ctypes.byref(n)))
        return ms.value, w.value, n.value

    def profile_families(self):
        """{family name: (ms, work, launches)} for every family with launches, after profile_end."""
        out = {}
        for name, k in PROF_KINDS.items():
            r = self.profile_kind(k)
            if r[2]:
                out[name] = r
        return out

    def tape_reset(self):
        _check(_lib.tfb_tape_reset(self.ptr))
        self._keep.clear()


def _out(ctx: Context, fn, *args) -> Tensor:
    h = c_int32()
    _check(fn(ctx.ptr, *args, ctypes.byref(h)))
    return Tensor(ctx, h.value)


# ------------------------------------------------------------------------- ops
OUT_BF16_COPY = 1
OUT_BF16_ONLY = 2


def add(a: Tensor, b: Tensor) -> Tensor:
    return _out(a.ctx, _lib.tfb_add, a.h, b.h)


def mul(a: Tensor, b: Tensor) -> Tensor:
    return _out(a.ctx, _lib.tfb_mul, a.h, b.h)


def scale(a: Tensor, s: float) -> Tensor:
    return _out(a.ctx, _lib.tfb_scale, a.h, c_float(s))


def sum_all(a: Tensor) -> Tensor:
    return _out(a.ctx, _lib.tfb_sum, a.h)


def reshape(a: Tensor, shape) -> Tensor:
    shape = tuple(int(s) for s in shape)
    return _out(a.ctx, _lib.tfb_reshape, a.h, _i64s(shape), len(shape))


def tanh(a: Tensor) -> Tensor:
    return _out(a.ctx, _lib.tfb_tanh, a.h)


def gelu(a: Tensor, bf16_only: bool = False) -> Tensor:
    """bf16_only (bf16 variant): only the output's bf16 copy is written, for an output
    that contractions read next; fp32 readers get it converted from those values."""
    if bf16_only:
        return _out(a.ctx, _lib.tfb_gelu_ex, a.h, OUT_BF16_ONLY)
    return _out(a.ctx, _lib.tfb_gelu, a.h)


def matmul(x: Tensor, w: Tensor) -> Tensor:
    return _out(x.ctx, _lib.tfb_matmul, x.h, w.h)


def matmul_t(x: Tensor, w: Tensor, bf16_only: bool = False) -> Tensor:
    """y = x @ w^T.  bf16_only: in the bf16 variant y is stored as bf16 alone (the
    cross-entropy reads such logits directly)."""
    if bf16_only:
        return _out(x.ctx, _lib.tfb_matmul_t_ex, x.h, w.h, OUT_BF16_ONLY)
    return _out(x.ctx, _lib.tfb_matmul_t, x.h, w.h)


def linear(x: Tensor, w: Tensor, b: Tensor, bf16_copy: bool = False, residual: Tensor = None,
           bf16_only: bool = False) -> Tensor:
    """x @ w + b (+ residual).  bf16_copy: the product also writes the output's bf16
    copy (bf16 variant), for an output that a contraction or the attention kernels
    read next; bf16_only: that copy alone.  residual: added in the product's
    epilogue (one op on the tape)."""
    if residual is not None:
        if bf16_copy or bf16_only:
            raise ValueError("linear: bf16 output options and residual are not combined")
        return _out(x.ctx, _lib.tfb_linear_residual, x.h, w.h, b.h, residual.h)
    if bf16_copy or bf16_only:
        return _out(x.ctx, _lib.tfb_linear_ex, x.h, w.h, b.h, OUT_BF16_ONLY if bf16_only else OUT_BF16_COPY)
    return _out(x.ctx, _lib.tfb_linear, x.h, w.h, b.h)


def layernorm(x: Tensor, gamma: Tensor, beta: Tensor, eps: float = 1e-5, bf16_only: bool = False) -> Tensor:
    """bf16_only: as for gelu."""
    if bf16_only:
        return _out(x.ctx, _lib.tfb_layernorm_ex, x.h, gamma.h, beta.h, c_float(eps), OUT_BF16_ONLY)
    return _out(x.ctx, _lib.tfb_layernorm, x.h, gamma.h, beta.h, c_float(eps))


def linear_gelu(x: Tensor, w: Tensor, b: Tensor, bf16_only: bool = False) -> Tensor:
    """Inference only: gelu(x @ w + b) as one call (in a product of at most 16 rows the
    GELU is applied where the partial products are summed)."""
    return _out(x.ctx, _lib.tfb_linear_gelu, x.h, w.h, b.h, OUT_BF16_ONLY if bf16_only else 0)


def linear_residual_layernorm(x: Tensor, w: Tensor, b: Tensor, residual: Tensor, gamma: Tensor, beta: Tensor,
                              eps: float = 1e-5, bf16_only: bool = False):
    """Inference only: (y, h) with y = residual + (x @ w + b) and h = LayerNorm(y) as one
    call (the few-row kernel's chunk sum adds the bias and residual and normalises each
    row).  bf16_only applies to h."""
    ctx = x.ctx
    y, h = c_int32(), c_int32()
    _check(_lib.tfb_linear_residual_layernorm(ctx.ptr, x.h, w.h, b.h, residual.h, gamma.h, beta.h, c_float(eps),
                                              OUT_BF16_ONLY if bf16_only else 0, ctypes.byref(y), ctypes.byref(h)))
    return Tensor(ctx, y.value), Tensor(ctx, h.value)


def mlp_residual_layernorm(x: Tensor, w_fc: Tensor, b_fc: Tensor, w_proj: Tensor, b_proj: Tensor, residual: Tensor,
                           gamma: Tensor, beta: Tensor, eps: float = 1e-5, bf16_only: bool = False):
    """Inference only: (y, h) with y = residual + gelu(x @ w_fc + b_fc) @ w_proj + b_proj and
    h = LayerNorm(y), as one call (the hidden activation is never stored for at most 16 rows)."""
    ctx = x.ctx
    y, h = c_int32(), c_int32()
    _check(_lib.tfb_mlp_residual_layernorm(ctx.ptr, x.h, w_fc.h, b_fc.h, w_proj.h, b_proj.h, residual.h, gamma.h,
                                           beta.h, c_float(eps), OUT_BF16_ONLY if bf16_only else 0, ctypes.byref(y),
                                           ctypes.byref(h)))
    return Tensor(ctx, y.value), Tensor(ctx, h.value)


def embedding(table: Tensor, ids, batch: int) -> Tensor:
    ctx = table.ctx
    d = ctx.device_ints(ids)
    return _out(ctx, _lib.tfb_embedding, table.h, c_void_p(d.data_ptr()), d.numel(), int(batch))


def narrow(x: Tensor, start: int, length: int) -> Tensor:
    return _out(x.ctx, _lib.tfb_narrow, x.h, int(start), int(length))


def split_heads(x: Tensor, heads: int) -> Tensor:
    return _out(x.ctx, _lib.tfb_split_heads, x.h, int(heads))


def merge_heads(x: Tensor) -> Tensor:
    return _out(x.ctx, _lib.tfb_merge_heads, x.h)


def batch_matmul(a: Tensor, b: Tensor) -> Tensor:
    return _out(a.ctx, _lib.tfb_batch_matmul, a.h, b.h)


def batch_matmul_t(a: Tensor, b: Tensor) -> Tensor:
    return _out(a.ctx, _lib.tfb_batch_matmul_t, a.h, b.h)


def causal_softmax(s: Tensor) -> Tensor:
    return _out(s.ctx, _lib.tfb_causal_softmax, s.h)


def causal_attention(qkv: Tensor, heads: int, bf16_only: bool = False) -> Tensor:
    """bf16_only: in the bf16 variant (fused kernels) the output is stored as bf16 alone."""
    if bf16_only:
        return _out(qkv.ctx, _lib.tfb_causal_attention_ex, qkv.h, int(heads), OUT_BF16_ONLY)
    return _out(qkv.ctx, _lib.tfb_causal_attention, qkv.h, int(heads))


CE_GRAD_BF16_ONLY = 1


def softmax_cross_entropy(logits: Tensor, targets, bf16_grad_only: bool = False) -> Tensor:
    """Mean cross-entropy of softmax(logits) against targets.  bf16_grad_only (bf16
    variant): logits produced by a contraction and read by nothing else get their
    gradient only as the bf16 copy that contraction's backward reads; logits.grad()
    is then unavailable."""
    ctx = logits.ctx
    d = ctx.device_ints(targets)
    if bf16_grad_only:
        return _out(ctx, _lib.tfb_softmax_cross_entropy_ex, logits.h, c_void_p(d.data_ptr()), d.numel(),
                    CE_GRAD_BF16_ONLY)
    return _out(ctx, _lib.tfb_softmax_cross_entropy, logits.h, c_void_p(d.data_ptr()), d.numel())


# ------------------------------------------------------------------------- optimizers
class AdamW:
    def __init__(self, params: Sequence[Tensor], lr: float, weight_decay: float = 0.01, beta1: float = 0.9,
                 beta2: float = 0.999, eps: float = 1e-8):
        self.ctx = params[0].ctx
        self.params = list(params)
        hs = (c_int32 * len(params))(*[p.h for p in params])
        ptr = c_void_p()
        _check(_lib.tfb_adamw_create(self.ctx.ptr, hs, len(params), c_float(lr), c_float(weight_decay),
                                     c_float(beta1), c_float(beta2), c_float(eps), ctypes.byref(ptr)))
        self.ptr = ptr

    def step(self):
        _check(_lib.tfb_adamw_step(self.ptr))

    def zero_grad(self):
        self.ctx.zero_grad(self.params)

    def set_lr(self, lr: float):
        _check(_lib.tfb_adamw_set_lr(self.ptr, c_float(lr)))

    def moments(self, i: int):
        n = self.params[i].size
        m = np.empty(self.params[i].shape, np.float32)
        v = np.empty(self.params[i].shape, np.float32)
        _check(_lib.tfb_adamw_moments(self.ptr, i, m.ctypes.data, v.ctypes.data, n))
        return m, v

    def close(self):
        if getattr(self, "ptr", None):
            _check(_lib.tfb_adamw_destroy(self.ptr))
            self.ptr = None


# ------------------------------------------------------------------------- KV-cached inference
class KvCache:
    def __init__(self, ctx: Context, layers: int, batch: int, tmax: int, channels: int):
        self.ctx = ctx
        ptr = c_void_p()
        _check(_lib.tfb_kv_create(ctx.ptr, layers, batch, tmax, channels, ctypes.byref(ptr)))
        self.ptr = ptr

    def store(self, layer: int, qkv: Tensor, pos0: int):
        _check(_lib.tfb_kv_store(self.ctx.ptr, self.ptr, layer, qkv.h, pos0))

    def attend(self, layer: int, qkv: Tensor, pos: int, heads: int) -> Tensor:
        return _out(self.ctx, _lib.tfb_kv_attend, self.ptr, layer, qkv.h, pos, heads)

    def attend_linear(self, layer: int, x: Tensor, w: Tensor, b: Tensor, pos: int, heads: int) -> Tensor:
        """The c_attn Linear (x @ w + b) and attend() as one call (inference)."""
        return _out(self.ctx, _lib.tfb_kv_attend_linear, self.ptr, layer, x.h, w.h, b.h, pos, heads)

    def attention_block(self, layer: int, x: Tensor, w_attn: Tensor, b_attn: Tensor, pos: int, heads: int,
                        w_proj: Tensor, b_proj: Tensor, residual: Tensor, gamma: Tensor, beta: Tensor,
                        eps: float = 1e-5, bf16_only: bool = False):
        """Inference only: (y, h) with y = residual + attend_linear(...) @ w_proj + b_proj and
        h = LayerNorm(y), as one call (the attention output is never stored where the
        fused kernels apply).  bf16_only applies to h."""
        y, h = c_int32(), c_int32()
        _check(_lib.tfb_kv_attention_block(self.ctx.ptr, self.ptr, layer, x.h, w_attn.h, b_attn.h, pos, heads,
                                           w_proj.h, b_proj.h, residual.h, gamma.h, beta.h, c_float(eps),
                                           OUT_BF16_ONLY if bf16_only else 0, ctypes.byref(y), ctypes.byref(h)))
        return Tensor(self.ctx, y.value), Tensor(self.ctx, h.value)

    def close(self):
        if getattr(self, "ptr", None):
            _check(_lib.tfb_kv_destroy(self.ptr))
            self.ptr = None


def sample_topk(logits: Tensor, k: int, temperature: float, uniforms, out=None):
    """uniforms: a float64 device tensor (one per row); returns an int32 device tensor of ids."""
    import torch
    ctx = logits.ctx
    rows = logits.size // logits.shape[-1]
    if out is None:
        out = torch.empty(rows, dtype=torch.int32, device=f"cuda:{ctx.device}")
    _check(_lib.tfb_sample_topk(ctx.ptr, logits.h, int(k), c_float(temperature), c_void_p(uniforms.data_ptr()),
                                c_void_p(out.data_ptr())))
    return out


def sgd_step(params: Sequence[Tensor], lr: float):
    ctx = params[0].ctx
    hs = (c_int32 * len(params))(*[p.h for p in params])
    _check(_lib.tfb_sgd_step(ctx.ptr, hs, len(params), c_float(lr)))
