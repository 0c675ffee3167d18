"""KV-cached inference through the C ABI against the oracle: the top-k /
temperature sampler, the per-step logits of generation (teacher-forced: the
oracle consumes the GPU's sampled tokens), the pages' invariant that the cached
path equals the full forward, and the inference workload at its own size
(16 prompts of 768 tokens, 256 sampled steps)."""
import numpy as np
import pytest

import synthetic as S
from oracle import decode as D
from oracle import engine as E
from oracle import models as M
from parity import FWD_TOL, assert_close, bf16_round

pytestmark = pytest.mark.gpu

T = pytest.importorskip("transformer_fwd_bwd_amd")
from transformer_fwd_bwd_amd import gpt as G  # noqa: E402


def near_boundary(probs, u, tol=1e-6):
    c = np.cumsum(probs)
    return np.min(np.abs(c - u)) < tol


def test_sampler_matches_oracle(ctx):
    import torch
    rng = S.rng_for(70)
    B, V = 6, 1000
    logits = rng.standard_normal((B, V)).astype(np.float32) * 3
    logits[0, :50] = 2.5           # a block of ties across the k-th value
    logits[1, :] = 0.0             # all equal
    u = rng.random(B)
    for k, temp in ((40, 1.0), (1, 1.0), (0, 0.7), (5, 2.0)):
        lt = ctx.tensor(logits.shape, logits)
        ud = torch.from_numpy(u).to("cuda:0")
        got = T.sample_topk(lt, k, temp, ud).cpu().numpy()
        for b in range(B):
            p = D.top_k_temperature_probs(logits[b].astype(np.float64), k, temp)
            want = D.sample(p, u[b])
            assert got[b] == want or near_boundary(p, u[b]), (k, b, got[b], want)
        lt.release()
        ctx.tape_reset()


def test_sampler_matches_oracle_vocab_rows(ctx):
    """Rows of 50,257 logits (the GPT-2 vocabulary): a plain cut at k = 40 and k = 500,
    a block of 600 ties straddling the k-th value, no cut (k = 0), a cut wider than the
    tie block (k = 1000), and a row whose top logit dominates."""
    import torch
    rng = S.rng_for(77)
    V = 50257
    cases = [(40, 1.0), (500, 0.8), (40, 1.0), (0, 1.0), (1000, 1.5), (40, 0.05)]
    B = len(cases)
    logits = (rng.standard_normal((B, V)) * 2).astype(np.float32)
    logits[2, rng.choice(V, 600, replace=False)] = 6.0      # 600 ties at the top: all survive k = 40
    logits[5, 123] = 40.0
    u = rng.random(B)
    lt = ctx.tensor(logits.shape, logits)
    for k, temp in {c for c in cases}:
        got = T.sample_topk(lt, k, temp, torch.from_numpy(u).to("cuda:0")).cpu().numpy()
        for b in range(B):
            p = D.top_k_temperature_probs(logits[b].astype(np.float64), k, temp)
            want = D.sample(p, u[b])
            assert got[b] == want or near_boundary(p, u[b]), (k, temp, b, got[b], want)
    lt.release()
    ctx.tape_reset()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
@pytest.mark.parametrize("hs,H", [(32, 4), (64, 3), (128, 2), (48, 2)])
def test_kv_attend_across_position_blocks(ctx, hs, H, prec):
    """[GPT2-4, "Generation with KV cache"]: one cached attention step of layer 1
    against the oracle's per-head softmax over every stored key, at positions on
    both sides of the blocks the step is split into (128 positions of an fp32
    cache, 256 of a bf16 one), at position 0 of a fresh cache (nothing stored
    yet), and at the last position of the cache.  Head size 48 takes the unsplit
    kernel.  A bf16 cache holds the keys and values rounded
    to nearest-even bf16; the oracle takes those same values, and the kernel's
    arithmetic on them is fp32, so both caches meet the fp32 tolerance."""
    from oracle import ops as O
    rng = S.rng_for(78 + hs)
    B, C, Tmax = 3, hs * H, 300
    ctx.set_precision(prec)
    kv = T.KvCache(ctx, 2, B, Tmax, C)
    cached = bf16_round if prec == "bf16" else (lambda a: a)
    K = np.zeros((B, Tmax, C)); Vv = np.zeros((B, Tmax, C))

    def store(p0, n):
        q = rng.standard_normal((B, n, 3 * C)).astype(np.float32)
        t = ctx.tensor(q.shape, q)
        kv.store(1, t, p0)
        K[:, p0:p0 + n] = cached(q[:, :, C:2 * C])
        Vv[:, p0:p0 + n] = cached(q[:, :, 2 * C:])
        t.release()

    try:
        for pos in (0, 126, 127, 128, 129, 255, 256, 257, 299):
            if pos == 126:
                store(0, 126)
            if pos > 130 and not K[:, pos - 1].any():
                store(130, pos - 130)
            q = rng.standard_normal((B, 1, 3 * C)).astype(np.float32)
            t = ctx.tensor(q.shape, q)
            y = kv.attend(1, t, pos, H).numpy().reshape(B, C)
            K[:, pos] = cached(q[:, 0, C:2 * C])
            Vv[:, pos] = cached(q[:, 0, 2 * C:])
            ref = np.zeros((B, C))
            for b in range(B):
                for h in range(H):
                    sl = slice(h * hs, (h + 1) * hs)
                    p = O.softmax_row(K[b, :pos + 1, sl] @ q[b, 0, sl].astype(np.float64) / np.sqrt(hs))
                    ref[b, sl] = p @ Vv[b, :pos + 1, sl]
            assert_close(y, ref, FWD_TOL["fp32"], f"pos {pos}")
            t.release()
            ctx.tape_reset()
    finally:
        kv.close()
        ctx.set_precision("fp32")


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_kv_cache_memory_returns_to_the_arena(ctx, prec):
    """Destroying a cache gives its memory back: repeated generations in one context do
    not grow the persistent arena, also in the bf16 variant, where the first generation
    makes the weights' bf16 copies after its cache (that cache then leaves a hole below
    them, which the next cache reuses); a cache followed by a parameter leaves a hole
    that the next allocation of its size takes."""
    import torch
    s, params, _ = S.tiny_gpt()
    ctx.set_precision(prec)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    prompts = torch.from_numpy(S.random_ids(79, (2, 5), s.vocab)).to("cuda:0")
    u = torch.from_numpy(S.rng_for(80).random((2, 3))).to("cuda:0")
    first = model.generate(prompts, 3, u, 5, 1.0).cpu().numpy()
    base = ctx.arena_usage()[0]
    for _ in range(3):
        again = model.generate(prompts, 3, u, 5, 1.0).cpu().numpy()
        assert ctx.arena_usage()[0] == base
        np.testing.assert_array_equal(again, first)
    kv = T.KvCache(ctx, 1, 2, 8, s.n_embd)
    held = ctx.arena_usage()[0]
    p = ctx.tensor((1 << 20,), param=True)               # larger than any hole: at the top
    top = ctx.arena_usage()[0]
    assert top > held >= base
    kv.close()
    assert ctx.arena_usage()[0] == top                   # below p: a hole, the top stays
    kv2 = T.KvCache(ctx, 1, 2, 8, s.n_embd)             # takes the hole the first one left
    assert ctx.arena_usage()[0] == top
    kv2.close()
    p.release()
    for t in model.param_list:
        t.release()
    ctx.set_precision("fp32")


def _teacher_forced(ctx, prec, B=4, Pn=16, steps=20, k=40, temp=1.0):
    import torch
    s, params, _ = S.tiny_gpt()
    ctx.set_precision(prec)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    prompts = S.random_ids(71, (B, Pn), s.vocab)
    u = S.rng_for(72).random((B, steps))
    seen = []
    toks = model.generate(torch.from_numpy(prompts).to("cuda:0"), steps, torch.from_numpy(u).to("cuda:0"), k, temp,
                          on_step=lambda i, lg, tk: seen.append(lg.numpy().reshape(B, -1)))
    toks = toks.cpu().numpy()
    # oracle: every prompt token then every sampled token through its own KV step
    P64 = {kk: v.astype(np.float64) for kk, v in params.items()}
    cache = D.KvCache(s.n_layer)
    for pos in range(Pn - 1):
        D.step(P64, prompts[:, pos], pos, cache, s.n_layer, s.n_head)
    tok = prompts[:, -1]
    for i in range(steps):
        ref = D.step(P64, tok, Pn - 1 + i, cache, s.n_layer, s.n_head)
        assert_close(seen[i], ref, FWD_TOL[prec], f"step {i} logits")
        for b in range(B):
            p = D.top_k_temperature_probs(ref[b], k, temp)
            want = D.sample(p, u[b, i])
            assert toks[b, i] == want or near_boundary(p, u[b, i]) or prec == "bf16", (i, b)
        tok = toks[:, i]
    for t in model.param_list:
        t.release()
    ctx.set_precision("fp32")
    return toks


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_generation_teacher_forced_tiny_gpt(ctx, prec):
    _teacher_forced(ctx, prec)


def test_kv_step_equals_full_forward(ctx):
    """[GPT2-4, "Generation with KV cache"]: the cached step's logits equal the
    full forward's logits at the same position."""
    import torch
    s, params, _ = S.tiny_gpt()
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    ids = S.random_ids(73, (3, 24), s.vocab)
    ctx.set_grad_enabled(False)
    full = model.logits(ids).numpy()
    ctx.tape_reset()
    kv = T.KvCache(ctx, s.n_layer, 3, 24, s.n_embd)
    ids_d = torch.from_numpy(ids).to("cuda:0")
    model.prefill(ids_d[:, :12].contiguous(), kv)
    ctx.tape_reset()
    for pos in range(12, 24):
        lg = model.decode_step(ids_d[:, pos].contiguous(), pos, kv, 24).numpy().reshape(3, -1)
        assert_close(lg, full[:, pos], 1e-5, f"pos {pos}")
        ctx.tape_reset()
    ctx.set_grad_enabled(True)
    kv.close()
    for t in model.param_list:
        t.release()


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_uncached_generation_equals_cached_at_every_step(ctx, prec):
    """[GPT2-4, "Generation with KV cache"]: generation without the cache (the whole
    forward per new token, sampled from the last position) against the cached path
    at every step -- same logits, same tokens -- and against the oracle's full forward
    over the sequence it sampled.  The sequences run up to the last position embedding."""
    import torch
    s, params, _ = S.tiny_gpt()
    ctx.set_precision(prec)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    B, Pn, k = 3, 9, 20
    steps = s.n_positions - Pn + 1                      # the last step's input is position n_positions - 1
    prompts = S.random_ids(74, (B, Pn), s.vocab)
    u = S.rng_for(75).random((B, steps))
    pd, ud = torch.from_numpy(prompts).to("cuda:0"), torch.from_numpy(u).to("cuda:0")
    cached, full = [], []
    tc = model.generate(pd, steps, ud, k, 1.0, on_step=lambda i, lg, tk: cached.append(lg.numpy().reshape(B, -1)))
    tu = model.generate_uncached(pd, steps, ud, k, 1.0, on_step=lambda i, lg, tk: full.append(lg.numpy().reshape(B, -1)))
    tc, tu = tc.cpu().numpy(), tu.cpu().numpy()
    assert tu.shape == (B, steps) and len(full) == steps
    seq = np.concatenate([prompts, tu[:, :-1]], axis=1)
    with E.no_grad():
        ref = M.gpt_logits(M.as_tensors(params), seq, s.n_layer, s.n_head).data
    for b in range(B):
        diff = np.flatnonzero(tc[b] != tu[b])
        same_until = diff[0] if diff.size else steps      # the two paths saw the same sequence up to here
        if prec == "fp32":
            assert same_until == steps or near_boundary(
                D.top_k_temperature_probs(ref[b, Pn - 1 + same_until], k, 1.0), u[b, same_until]), (b, same_until)
        for i in range(steps):
            assert_close(full[i][b], ref[b, Pn - 1 + i], FWD_TOL[prec], f"uncached step {i} row {b}")
            if i <= same_until and i < steps:
                assert_close(full[i][b], cached[i][b], FWD_TOL[prec], f"uncached vs cached step {i} row {b}")
            p = D.top_k_temperature_probs(ref[b, Pn - 1 + i], k, 1.0)
            assert tu[b, i] == D.sample(p, u[b, i]) or near_boundary(p, u[b, i]) or prec == "bf16", (b, i)
    with pytest.raises(ValueError):
        model.generate_uncached(pd, steps + 1, torch.from_numpy(S.rng_for(76).random((B, steps + 1))).to("cuda:0"),
                                k, 1.0)
    with pytest.raises(ValueError):
        model.generate(pd, steps + 1, torch.from_numpy(S.rng_for(76).random((B, steps + 1))).to("cuda:0"), k, 1.0)
    for t in model.param_list:
        t.release()
    ctx.set_precision("fp32")


@pytest.mark.parametrize("prec", ["fp32", "bf16"])
def test_inference_workload_gpt2_shape(ctx, prec):
    """16 prompts x 768 tokens, then 256 sampled steps (top-k 40, temperature 1)
    at the GPT-2-124M shape, in both variants; sampled steps of sequence 5 against
    the oracle's full forward over that sequence's prompt and the GPU's sampled
    tokens (teacher-forced: in the bf16 variant the sampled tokens may part from
    the oracle's own draws, so the logits are compared on the sequence the GPU
    generated).  In bf16 this is the 16-row product that rounds its input as it
    loads it, the split cached attention and the register-resident sampler."""
    import torch
    s, params, prompts, u = S.gpt2_infer()
    B, Pn = prompts.shape
    steps = u.shape[1]
    big = T.Context(arena_bytes=16 << 30, precision=prec)
    model = G.Gpt(big, s.n_layer, s.n_head, params)
    b, check = 5, (0, 1, 128, 255)
    seen = {}

    def on_step(i, lg, tk):
        if i in check:
            seen[i] = lg.numpy().reshape(B, -1)[b]
    toks = model.generate(torch.from_numpy(prompts).to("cuda:0"), steps, torch.from_numpy(u).to("cuda:0"), 40, 1.0,
                          on_step=on_step).cpu().numpy()
    assert toks.shape == (B, steps) and toks.min() >= 0 and toks.max() < s.vocab
    seq = np.concatenate([prompts[b], toks[b, :-1]])[None, :]          # 1023 positions
    with E.no_grad():
        ref = M.gpt_logits(M.as_tensors(params), seq, s.n_layer, s.n_head).data[0]
    for i in check:
        r = ref[Pn - 1 + i]
        assert_close(seen[i], r, FWD_TOL[prec], f"step {i}")
        if prec == "fp32":
            p = D.top_k_temperature_probs(r, 40, 1.0)
            assert toks[b, i] == D.sample(p, u[b, i]) or near_boundary(p, u[b, i]), i
    big.close()
