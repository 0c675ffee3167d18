"""Forward and backward rule of every tensor op, as plain definitions.

Test infrastructure only (see the package docstring).  Every function takes and
returns numpy arrays; arithmetic happens in the dtype of the inputs (float64 for
parity, float32 only where a pin reproduces the pages' own float arithmetic).
Backward functions return the contribution to each input's gradient; the engine
adds it (the "+=" rule of [Autograd-1, §"Why += and not ="]).

Shapes follow [Autograd-1, §"The Tensor class"]: flat row-major data; a tensor's
"rows" are the product of all but the last dimension.
"""
from __future__ import annotations

import math

import numpy as np


def _rows(a: np.ndarray) -> np.ndarray:
    return a.reshape(-1, a.shape[-1])


# --------------------------------------------------------------------------
# Elementwise and shape ops  [Autograd-1, §"Ops" and the table of remaining ops]
# --------------------------------------------------------------------------
def add_fwd(a, b):
    """a + b, where b equals a's trailing dimensions (the bias broadcast)."""
    if a.shape[a.ndim - b.ndim:] != b.shape:
        raise ValueError(f"add: {b.shape} does not match the trailing dims of {a.shape}")
    return a + b


def add_bwd(g, a_shape, b_shape):
    """da = g; db = g summed over the broadcast (leading) dimensions."""
    lead = len(a_shape) - len(b_shape)
    db = g.sum(axis=tuple(range(lead))) if lead else g.copy()
    return g.copy(), db


def mul_fwd(a, b):
    if a.size != b.size:
        raise ValueError("mul: sizes differ")
    return a * b


def mul_bwd(g, a, b):
    """d(a*b)/da = b, d(a*b)/db = a."""
    return g * b, g * a


def scale_fwd(a, s):
    return a * s


def scale_bwd(g, s):
    return g * s


def sum_fwd(a):
    return np.array([a.sum()], dtype=a.dtype)


def sum_bwd(g, shape):
    return np.full(shape, g[0], dtype=g.dtype)


def tanh_fwd(x):
    return np.tanh(x)


def tanh_bwd(g, y):
    """tanh'(x) = 1 - tanh(x)^2, written with the saved output y."""
    return g * (1 - y * y)


GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715


def gelu_fwd(x):
    """tanh approximation of GELU (GPT-2's "gelu_new"; [GPT2-4, §"Common mistakes"]):
    0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    u = GELU_C * (x + GELU_A * x ** 3)
    return 0.5 * x * (1 + np.tanh(u))


def gelu_bwd(g, x):
    u = GELU_C * (x + GELU_A * x ** 3)
    t = np.tanh(u)
    du = GELU_C * (1 + 3 * GELU_A * x * x)
    return g * (0.5 * (1 + t) + 0.5 * x * (1 - t * t) * du)


# --------------------------------------------------------------------------
# MatMul family  [Autograd-1, §"Ops": MatMul and the gradient shapes]
# --------------------------------------------------------------------------
def matmul_fwd(x, w):
    """x[..., K] @ w[K, M] -> [..., M] (leading dims of x flattened to rows)."""
    if w.ndim != 2 or w.shape[0] != x.shape[-1]:
        raise ValueError(f"matmul {x.shape} @ {w.shape}")
    return (_rows(x) @ w).reshape(*x.shape[:-1], w.shape[1])


def matmul_bwd(g, x, w):
    """dx = g @ w^T, dw = x^T @ g."""
    g2 = _rows(g)
    dx = (g2 @ w.T).reshape(x.shape)
    dw = _rows(x).T @ g2
    return dx, dw


def matmul_t_fwd(x, w):
    """x[..., C] @ w[V, C]^T -> [..., V]; the weight-tied LM head ([GPT2-4, §"Loading the weights"])."""
    if w.ndim != 2 or w.shape[1] != x.shape[-1]:
        raise ValueError(f"matmul_t {x.shape} @ {w.shape}^T")
    return (_rows(x) @ w.T).reshape(*x.shape[:-1], w.shape[0])


def matmul_t_bwd(g, x, w):
    """dx = g @ w, dw = g^T @ x."""
    g2 = _rows(g)
    dx = (g2 @ w).reshape(x.shape)
    dw = g2.T @ _rows(x)
    return dx, dw


def batch_matmul_fwd(a, b):
    """a[Z, n, k] @ b[Z, k, m] per batch entry."""
    return np.matmul(a, b)


def batch_matmul_bwd(g, a, b):
    return np.matmul(g, np.swapaxes(b, -1, -2)), np.matmul(np.swapaxes(a, -1, -2), g)


def batch_matmul_t_fwd(a, b):
    """a[Z, n, k] @ b[Z, m, k]^T per batch entry."""
    return np.matmul(a, np.swapaxes(b, -1, -2))


def batch_matmul_t_bwd(g, a, b):
    return np.matmul(g, b), np.matmul(np.swapaxes(g, -1, -2), a)


# --------------------------------------------------------------------------
# Embedding, LayerNorm  [Autograd-1, table of ops; GPT2-4, §"Generation with KV cache"]
# --------------------------------------------------------------------------
def embedding_fwd(table, ids, batch):
    """Row gather: out[b, t, :] = table[ids[b*T + t], :], T = len(ids) / batch."""
    ids = np.asarray(ids).reshape(-1)
    if ids.size % batch:
        raise ValueError("embedding: ids not divisible by batch")
    if ids.min(initial=0) < 0 or ids.max(initial=0) >= table.shape[0]:
        raise IndexError("embedding: id out of range")
    return table[ids].reshape(batch, ids.size // batch, table.shape[1])


def embedding_bwd(g, ids, table_shape):
    """Scatter-add of the output rows' gradients into the rows they were read from."""
    ids = np.asarray(ids).reshape(-1)
    d = np.zeros(table_shape, dtype=g.dtype)
    np.add.at(d, ids, _rows(g))
    return d


LN_EPS = 1e-5


def layernorm_fwd(x, gamma, beta, eps=LN_EPS):
    """Per row over the last dim: mean, biased variance, xhat = (x-mu)/sqrt(var+eps),
    y = gamma*xhat + beta.  Returns y and the saved (mean, rstd)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * rstd
    return gamma * xhat + beta, mu, rstd


def layernorm_bwd(g, x, gamma, mu, rstd):
    """Derivative of the definition above.  With dxhat = g*gamma:
    dx = rstd * (dxhat - mean(dxhat) - xhat * mean(dxhat * xhat)),
    dgamma = sum over rows of g*xhat, dbeta = sum over rows of g."""
    xhat = (x - mu) * rstd
    dxhat = g * gamma
    m1 = dxhat.mean(axis=-1, keepdims=True)
    m2 = (dxhat * xhat).mean(axis=-1, keepdims=True)
    dx = rstd * (dxhat - m1 - xhat * m2)
    lead = tuple(range(x.ndim - 1))
    return dx, (g * xhat).sum(axis=lead), g.sum(axis=lead)


# --------------------------------------------------------------------------
# Softmax family  [Autograd-1, §"Ops": SoftmaxCrossEntropy and Softmax]
# --------------------------------------------------------------------------
def softmax_row(x, temperature=1.0):
    """Max-subtracted softmax of one row: exp((x - max)/T) / sum."""
    m = np.max(x)
    e = np.exp((x - m) / temperature)
    return e / e.sum()


def softmax_ce_fwd(logits, targets):
    """Row softmax, loss_r = -log(max(p[target_r], 1e-30)), loss = mean over rows.
    Returns (loss [1], probs)."""
    L = _rows(logits)
    targets = np.asarray(targets).reshape(-1)
    if targets.size != L.shape[0]:
        raise ValueError("one target per row")
    m = L.max(axis=1, keepdims=True)
    e = np.exp(L - m)
    p = e / e.sum(axis=1, keepdims=True)
    pt = p[np.arange(L.shape[0]), targets]
    losses = -np.log(np.maximum(pt, 1e-30))
    return np.array([losses.mean()], dtype=logits.dtype), p.reshape(logits.shape)


def softmax_ce_bwd(g, probs, targets):
    """dlogits = (g/n) * (p - onehot(target))."""
    P = _rows(probs)
    n = P.shape[0]
    d = P * (g[0] / n)
    d[np.arange(n), np.asarray(targets).reshape(-1)] -= g[0] / n
    return d.reshape(probs.shape)


def causal_mask(rows, T):
    """Row r of a [rows, T] view sees columns j < (r mod T) + 1 ([GPT2-4, §"The 12 unused tensors"])."""
    r = np.arange(rows)[:, None] % T
    return np.arange(T)[None, :] <= r


def causal_softmax_fwd(s):
    """Softmax over the visible prefix of every row; masked entries are exactly 0."""
    T = s.shape[-1]
    S = _rows(s)
    vis = causal_mask(S.shape[0], T)
    z = np.where(vis, S, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.where(vis, np.exp(z - m), 0.0)
    return (e / e.sum(axis=1, keepdims=True)).reshape(s.shape)


def causal_softmax_bwd(g, p):
    """dS_j = P_j (dP_j - sum_k P_k dP_k) on visible j, 0 elsewhere (P is 0 there)."""
    G, P = _rows(g), _rows(p)
    inner = (G * P).sum(axis=1, keepdims=True)
    return (P * (G - inner)).reshape(p.shape)


# --------------------------------------------------------------------------
# Head plumbing  [Autograd-1, table of ops: Narrow, SplitHeads, MergeHeads]
# --------------------------------------------------------------------------
def narrow_fwd(x, start, length):
    """Slice of the last dimension."""
    if start < 0 or start + length > x.shape[-1]:
        raise ValueError("narrow out of range")
    return x[..., start:start + length].copy()


def narrow_bwd(g, x_shape, start):
    d = np.zeros(x_shape, dtype=g.dtype)
    d[..., start:start + g.shape[-1]] = g
    return d


def split_heads_fwd(x, heads):
    """[B, T, H*hs] -> [B, H, T, hs]; head h is columns h*hs .. h*hs+hs-1
    ([GPT2-4, §"Generation with KV cache": the per-head slice of q])."""
    B, T, C = x.shape
    return x.reshape(B, T, heads, C // heads).transpose(0, 2, 1, 3).copy()


def split_heads_bwd(g):
    B, H, T, hs = g.shape
    return g.transpose(0, 2, 1, 3).reshape(B, T, H * hs).copy()


def merge_heads_fwd(x):
    return split_heads_bwd(x)


def merge_heads_bwd(g, heads):
    return split_heads_fwd(g, heads)
