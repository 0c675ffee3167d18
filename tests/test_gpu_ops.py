"""Per-op parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs, forward values and every input gradient.  Sizes span
several 128-wide tiles and leave ragged tails in every dimension."""
import math

import numpy as np
import pytest

import synthetic as S
from oracle import engine as E
from parity import FWD_TOL, GRAD_TOL, assert_close, bf16_round as _bf16_round, gpu_op_with_grads, oracle_op_with_grads

pytestmark = pytest.mark.gpu

T = pytest.importorskip("transformer_fwd_bwd_amd")


def rnd(seed, shape, scale=1.0):
    return S.random_array(seed, shape, scale)


def check(ctx, prec, gpu_build, oracle_build, arrays, out_shape, seed=999, fwd_tol=None, grad_tol=None):
    ctx.set_precision(prec)
    R = rnd(seed, out_shape)
    out, grads = gpu_op_with_grads(ctx, gpu_build, arrays, R)
    ref, rgrads = oracle_op_with_grads(oracle_build, arrays, R)
    assert_close(out, ref, fwd_tol or FWD_TOL[prec], "forward")
    for i, (g, r) in enumerate(zip(grads, rgrads)):
        assert_close(g, r, grad_tol or GRAD_TOL[prec], f"grad {i}")
    ctx.set_precision("fp32")


PRECS = ["fp32", "bf16"]


@pytest.mark.parametrize("prec", PRECS)
def test_matmul(ctx, prec):
    check(ctx, prec, T.matmul, E.matmul, [rnd(1, (3, 100, 200)), rnd(2, (200, 260), 0.1)], (3, 100, 260))


@pytest.mark.parametrize("prec", PRECS)
def test_matmul_t(ctx, prec):
    check(ctx, prec, T.matmul_t, E.matmul_t, [rnd(3, (300, 200)), rnd(4, (261, 200), 0.1)], (300, 261))


@pytest.mark.parametrize("prec", PRECS)
def test_linear_is_matmul_plus_bias(ctx, prec):
    check(ctx, prec, T.linear, lambda x, w, b: E.add(E.matmul(x, w), b),
          [rnd(5, (300, 200)), rnd(6, (200, 260), 0.1), rnd(7, (260,))], (300, 260))


@pytest.mark.parametrize("prec", PRECS)
def test_linear_with_residual(ctx, prec):
    """[Autograd-1, "Ops": MatMul, bias Add, Add]: r + (x @ w + b) as one op, ragged in
    every dimension, against the oracle's three ops; every input's gradient."""
    def gpu(x, w, b, r):
        return T.linear(x, w, b, residual=r)

    def ora(x, w, b, r):
        return E.add(r, E.add(E.matmul(x, w), b))
    check(ctx, prec, gpu, ora, [rnd(111, (3, 100, 200)), rnd(112, (200, 260), 0.1), rnd(113, (260,)),
                                rnd(114, (3, 100, 260))], (3, 100, 260))


@pytest.mark.parametrize("prec", PRECS)
def test_linear_residual_is_input(ctx, prec):
    """The residual is the product's own input: both gradient contributions reach it."""
    def gpu(x, w, b):
        return T.linear(x, w, b, residual=x)

    def ora(x, w, b):
        return E.add(x, E.add(E.matmul(x, w), b))
    check(ctx, prec, gpu, ora, [rnd(115, (150, 96)), rnd(116, (96, 96), 0.1), rnd(117, (96,))], (150, 96))


@pytest.mark.parametrize("N", [128, 130])
def test_linear_residual_long_k_split(ctx, N):
    """A long reduction takes the K-split path: the residual is added by the split
    reduction (float4 and element forms)."""
    def gpu(x, w, b, r):
        return T.linear(x, w, b, residual=r)

    def ora(x, w, b, r):
        return E.add(r, E.add(E.matmul(x, w), b))
    check(ctx, "fp32", gpu, ora, [rnd(118, (200, 3000)), rnd(119, (3000, N), 0.02), rnd(120, (N,)),
                                  rnd(121, (200, N))], (200, N))


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,N", [(1, 3, 4), (5, 130, 132), (16, 768, 2304), (7, 3100, 68), (16, 256, 1028),
                                   (17, 300, 132), (5, 130, 130), (3, 70, 6)])
def test_linear_few_rows(ctx, prec, M, K, N):
    """Products of at most 16 rows (one token per sequence) take the small-row kernel:
    one k chunk, several chunks summed by the separate chunk-sum pass (gemv_reduce_k),
    ragged column strips; 17 rows take the tiled kernel, and so do few-row products
    whose column count is not a multiple of 4 (rows of w, b, r and y then sit off
    16-byte alignment), which in the bf16 variant read the fp32 input and round it
    as they load it.  r + (x @ w + b) and every gradient."""
    def gpu(x, w, b, r):
        return T.linear(x, w, b, residual=r)

    def ora(x, w, b, r):
        return E.add(r, E.add(E.matmul(x, w), b))
    check(ctx, prec, gpu, ora, [rnd(130 + M, (M, K)), rnd(131 + K, (K, N), 1 / np.sqrt(K)), rnd(132, (N,)),
                                rnd(133, (M, N))], (M, N))


def _infer(ctx, prec, arrays, build):
    ctx.set_precision(prec)
    ts = [ctx.tensor(a.shape, a) for a in arrays]
    ctx.set_grad_enabled(False)
    try:
        outs = build(*ts)
        outs = outs if isinstance(outs, tuple) else (outs,)
        res = [o.numpy() for o in outs]
    finally:
        ctx.set_grad_enabled(True)
        ctx.tape_reset()
        for t in ts:
            t.release()
        ctx.set_precision("fp32")
    return res


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,N", [(16, 768, 3072), (1, 128, 64), (3, 200, 132), (5, 64, 18), (20, 100, 96)])
def test_linear_gelu_inference(ctx, prec, M, K, N):
    """[GPT2-4, "Loading the weights": c_fc then GELU] gelu(x @ w + b) as one inference
    call: the GELU in the few-row kernel's chunk sum (several chunks), in its single-chunk
    epilogue (K = 128), and through the separate ops where that kernel does not take the
    product (18 columns; 20 rows)."""
    arrays = [rnd(170 + M, (M, K)), rnd(171 + K, (K, N), 1 / np.sqrt(K)), rnd(172, (N,), 0.5)]
    (y,) = _infer(ctx, prec, arrays, lambda x, w, b: T.linear_gelu(x, w, b, bf16_only=True))
    x, w, b = (a.astype(np.float64) for a in arrays)
    from oracle import ops as O
    assert_close(y, O.gelu_fwd(x @ w + b), FWD_TOL[prec], "gelu(x @ w + b)")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,N", [(16, 768, 768), (16, 3072, 768), (4, 64, 64), (5, 130, 132), (5, 130, 130),
                                   (20, 100, 96)])
def test_linear_residual_layernorm_inference(ctx, prec, M, K, N):
    """[GPT2-4, "Loading the weights": x = x + proj(.), then the next LayerNorm]
    y = r + (x @ w + b) and h = LayerNorm(y) as one inference call: normalised in the
    few-row kernel's chunk sum (6 and 24 chunks; one chunk), and through the separate ops
    where that kernel does not take the product (130 columns; 20 rows)."""
    arrays = [rnd(180 + M, (M, K)), rnd(181 + K, (K, N), 1 / np.sqrt(K)), rnd(182, (N,), 0.5), rnd(183, (M, N)),
              1 + rnd(184, (N,), 0.2), rnd(185, (N,), 0.2)]
    y, h = _infer(ctx, prec, arrays, lambda x, w, b, r, g, bt: T.linear_residual_layernorm(x, w, b, r, g, bt,
                                                                                            bf16_only=True))
    x, w, b, r, g, bt = (a.astype(np.float64) for a in arrays)
    from oracle import ops as O
    ry = r + x @ w + b
    rh = O.layernorm_fwd(ry, g, bt)[0]
    assert_close(y, ry, FWD_TOL[prec], "y")
    assert_close(h, rh, FWD_TOL[prec], "LayerNorm(y)")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("M,K,F", [(16, 768, 3072), (3, 64, 256), (20, 64, 128)])
def test_mlp_residual_layernorm_inference(ctx, prec, M, K, F):
    """[GPT2-4, "Loading the weights": x = x + mlp(ln_2(x)), then the next LayerNorm]
    y = r + gelu(x @ w1 + b1) @ w2 + b2 and h = LayerNorm(y) as one inference call: the
    projection sums the c_fc partials (6 chunks; 1 chunk) and applies the GELU as it
    loads them; 20 rows take the separate ops."""
    arrays = [rnd(190 + M, (M, K)), rnd(191, (K, F), 1 / np.sqrt(K)), rnd(192, (F,), 0.5),
              rnd(193, (F, K), 1 / np.sqrt(F)), rnd(194, (K,), 0.5), rnd(195, (M, K)), 1 + rnd(196, (K,), 0.2),
              rnd(197, (K,), 0.2)]
    y, h = _infer(ctx, prec, arrays, lambda *t: T.mlp_residual_layernorm(*t, bf16_only=True))
    x, w1, b1, w2, b2, r, g, bt = (a.astype(np.float64) for a in arrays)
    from oracle import ops as O
    ry = r + O.gelu_fwd(x @ w1 + b1) @ w2 + b2
    assert_close(y, ry, FWD_TOL[prec], "y")
    assert_close(h, O.layernorm_fwd(ry, g, bt)[0], FWD_TOL[prec], "LayerNorm(y)")


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("hs,H", [(64, 3), (48, 2)])
def test_kv_attend_linear(ctx, prec, hs, H):
    """[GPT2-4, "Generation with KV cache"] the c_attn Linear and the cached attention as
    one call, at positions on both sides of a 128-position block: the attention sums the
    product's partials as it reads q, k, v (head size 64) or runs after the stored
    product (head size 48); the next call must see the key and value it appended."""
    from oracle import ops as O
    ctx.set_precision(prec)
    rng = S.rng_for(200 + hs)
    B, C, K, Tmax = 4, hs * H, 96, 200
    kv = T.KvCache(ctx, 2, B, Tmax, C)
    Kc, Vc = np.zeros((B, Tmax, C)), np.zeros((B, Tmax, C))
    pre = rng.standard_normal((B, 127, 3 * C)).astype(np.float32)
    tq = ctx.tensor(pre.shape, pre)
    kv.store(1, tq, 0)
    Kc[:, :127], Vc[:, :127] = pre[:, :, C:2 * C], pre[:, :, 2 * C:]
    tq.release()
    w = rnd(201, (K, 3 * C), 1 / np.sqrt(K))
    b = rnd(202, (3 * C,), 0.3)
    tw, tb = ctx.tensor(w.shape, w), ctx.tensor(b.shape, b)
    ctx.set_grad_enabled(False)
    try:
        for pos in (127, 128, 129):
            x = rnd(203 + pos, (B, 1, K))
            tx = ctx.tensor(x.shape, x)
            y = kv.attend_linear(1, tx, tw, tb, pos, H).numpy().reshape(B, C)
            qkv = x.reshape(B, K).astype(np.float64) @ w + b
            Kc[:, pos], Vc[:, pos] = qkv[:, C:2 * C], qkv[:, 2 * C:]
            ref = np.zeros((B, C))
            for bb in range(B):
                for h in range(H):
                    sl = slice(h * hs, (h + 1) * hs)
                    p = O.softmax_row(Kc[bb, :pos + 1, sl] @ qkv[bb, sl] / np.sqrt(hs))
                    ref[bb, sl] = p @ Vc[bb, :pos + 1, sl]
            assert_close(y, ref, FWD_TOL[prec], f"pos {pos}")
            ctx.tape_reset()
            tx.release()
    finally:
        ctx.set_grad_enabled(True)
        ctx.set_precision("fp32")
    kv.close()
    tw.release()
    tb.release()


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("hs,H", [(64, 3), (48, 2)])
@pytest.mark.parametrize("P0", [254, 1022, 2310])
def test_kv_attention_block(ctx, prec, hs, H, P0):
    """[GPT2-4, "Generation with KV cache"; "Loading the weights": x = x + attn(ln_1(x))]
    the attention half of a block in one call -- c_attn, the cached attention, the
    projection plus the residual, and ln_2 -- at positions P0..P0+3 after P0 cached
    ones (head size 64: the projection merges the attention's per-block results as
    it loads them; head size 48: the unfused ops); each call must see the keys and
    values the previous ones appended.  Position 256 is a block boundary of either
    cache; at 1024 an fp32 cache goes from 8 blocks, the most the merge loads at
    once, to 9; past 2048 both caches take the merge's block-by-block loop."""
    from oracle import ops as O
    ctx.set_precision(prec)
    rng = S.rng_for(300 + hs)
    B, C, K = 4, hs * H, 96
    Tmax = P0 + 46
    kv = T.KvCache(ctx, 2, B, Tmax, C)
    Kc, Vc = np.zeros((B, Tmax, C)), np.zeros((B, Tmax, C))
    pre = rng.standard_normal((B, P0, 3 * C)).astype(np.float32)
    tq = ctx.tensor(pre.shape, pre)
    kv.store(1, tq, 0)
    Kc[:, :P0], Vc[:, :P0] = pre[:, :, C:2 * C], pre[:, :, 2 * C:]
    tq.release()
    w = rnd(301, (K, 3 * C), 1 / np.sqrt(K))
    b = rnd(302, (3 * C,), 0.3)
    wp = rnd(303, (C, C), 1 / np.sqrt(C))
    bp = rnd(304, (C,), 0.3)
    g = 1.0 + rnd(305, (C,), 0.2)
    bt = rnd(306, (C,), 0.2)
    held = [ctx.tensor(a.shape, a) for a in (w, b, wp, bp, g, bt)]
    tw, tb, twp, tbp, tg, tbt = held
    ctx.set_grad_enabled(False)
    try:
        for pos in range(P0, P0 + 4):
            x = rnd(307 + pos, (B, 1, K))
            r = rnd(407 + pos, (B, 1, C))
            tx, tr = ctx.tensor(x.shape, x), ctx.tensor(r.shape, r)
            ty, th = kv.attention_block(1, tx, tw, tb, pos, H, twp, tbp, tr, tg, tbt)
            y, h = ty.numpy().reshape(B, C), th.numpy().reshape(B, C)
            qkv = x.reshape(B, K).astype(np.float64) @ w + b
            Kc[:, pos], Vc[:, pos] = qkv[:, C:2 * C], qkv[:, 2 * C:]
            a = np.zeros((B, C))
            for bb in range(B):
                for hd in range(H):
                    sl = slice(hd * hs, (hd + 1) * hs)
                    p = O.softmax_row(Kc[bb, :pos + 1, sl] @ qkv[bb, sl] / np.sqrt(hs))
                    a[bb, sl] = p @ Vc[bb, :pos + 1, sl]
            ry = r.reshape(B, C) + a @ wp + bp
            assert_close(y, ry, FWD_TOL[prec], f"y, pos {pos}")
            assert_close(h, O.layernorm_fwd(ry, g, bt)[0], FWD_TOL[prec], f"ln_2(y), pos {pos}")
            ctx.tape_reset()
            tx.release()
            tr.release()
    finally:
        ctx.set_grad_enabled(True)
        ctx.set_precision("fp32")
        kv.close()
        for t in held:
            t.release()


def test_kv_attention_block_rejects_bad_shapes(ctx):
    """The fused attention block checks its operands before launching anything:
    a projection whose rows are not the cache's channels, a residual of another
    width, a position past the cache and a head count that does not divide the
    channels are shape errors; a cache of another context is an argument error."""
    B, C, K, Tmax = 2, 64, 32, 16
    kv = T.KvCache(ctx, 1, B, Tmax, C)
    made = []

    def mk(*shape):
        made.append(ctx.tensor(shape, rnd(len(shape) + sum(shape), shape)))
        return made[-1]

    x, wa, ba = mk(B, 1, K), mk(K, 3 * C), mk(3 * C)
    wp, bp, r, g, bt = mk(C, C), mk(C), mk(B, 1, C), mk(C), mk(C)
    ctx.set_grad_enabled(False)
    try:
        cases = [
            ("projection rows", lambda: kv.attention_block(0, x, wa, ba, 0, 2, mk(C + 4, C), bp, r, g, bt), -2),
            ("residual width", lambda: kv.attention_block(0, x, wa, ba, 0, 2, wp, bp, mk(B, 1, C + 4), g, bt), -2),
            ("position", lambda: kv.attention_block(0, x, wa, ba, Tmax, 2, wp, bp, r, g, bt), -2),
            ("heads", lambda: kv.attention_block(0, x, wa, ba, 0, 3, wp, bp, r, g, bt), -2),
            ("layer", lambda: kv.attention_block(1, x, wa, ba, 0, 2, wp, bp, r, g, bt), -1),
        ]
        for what, call, code in cases:
            with pytest.raises(T.TfbError) as e:
                call()
            assert e.value.code == code, (what, e.value.code, str(e.value))
        # the cache is untouched by the rejected calls: a good call still matches
        y, h = kv.attention_block(0, x, wa, ba, 0, 2, wp, bp, r, g, bt)
        assert np.isfinite(y.numpy()).all() and np.isfinite(h.numpy()).all()
    finally:
        ctx.set_grad_enabled(True)
        kv.close()
        ctx.tape_reset()
        for t in made:
            t.release()


def test_inference_fusions_refuse_to_record(ctx):
    x, w, b = ctx.tensor((2, 8), np.ones((2, 8), np.float32)), ctx.tensor((8, 8)), ctx.tensor((8,))
    with pytest.raises(T.TfbError) as e:
        T.linear_gelu(x, w, b)
    assert e.value.code == -3 and "inference-only" in str(e.value)
    with pytest.raises(T.TfbError) as e:
        T.linear_residual_layernorm(x, w, b, x, b, b)
    assert e.value.code == -3
    kv = T.KvCache(ctx, 1, 2, 8, 8)
    x1, wa, ba = ctx.tensor((2, 1, 8)), ctx.tensor((8, 24)), ctx.tensor((24,))
    with pytest.raises(T.TfbError) as e:
        kv.attention_block(0, x1, wa, ba, 0, 1, w, b, x1, b, b)
    assert e.value.code == -3 and "inference-only" in str(e.value)
    kv.close()
    ctx.tape_reset()
    for t in (x, w, b, x1, wa, ba):
        t.release()


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("V", [130, 1030])
def test_matmul_t_few_rows_accumulating_grad(ctx, prec, V):
    """x [5, 64] read by two products x @ w^T: the input gradient g @ w of each is a
    few-row product, the second added onto the first (beta = 1); with 1030 rows of w
    the output's rows are padded, so g is read at its padded stride."""
    def gpu(x, w1, w2):
        return T.add(T.matmul_t(x, w1), T.matmul_t(x, w2))

    def ora(x, w1, w2):
        return E.add(E.matmul_t(x, w1), E.matmul_t(x, w2))
    check(ctx, prec, gpu, ora, [rnd(150, (5, 64)), rnd(151, (V, 64), 0.1), rnd(152, (V, 64), 0.1)], (5, V))


@pytest.mark.parametrize("M,K,N", [(16, 768, 2304), (16, 3072, 768), (3, 130, 132), (17, 300, 132), (5, 130, 130),
                                   (16, 64, 18)])
def test_linear_few_rows_bf16_operands_exact(ctx, M, K, N):
    """In the bf16 variant a product multiplies the bf16 values of its operands exactly
    and accumulates in fp32: against the float64 product of the rounded operands the
    forward output differs only by fp32 accumulation (checked to 1e-5, far inside the
    bf16 tolerance, so a mishandled operand or a lost partial sum cannot hide)."""
    ctx.set_precision("bf16")
    x, w, b = rnd(140, (M, K)), rnd(141, (K, N), 1 / np.sqrt(K)), rnd(142, (N,))
    ts = [ctx.tensor(a.shape, a) for a in (x, w, b)]
    y = T.linear(*ts).numpy()
    ref = _bf16_round(x).astype(np.float64) @ _bf16_round(w).astype(np.float64) + b
    assert_close(y, ref, 1e-5, "forward")
    ctx.tape_reset()
    # kept as bf16 alone: the exact bf16 rounding of the plain output
    yb = T.linear(*ts, bf16_only=True).numpy()
    np.testing.assert_array_equal(yb, _bf16_round(y))
    ctx.tape_reset()
    for t in ts:
        t.release()
    ctx.set_precision("fp32")


@pytest.mark.parametrize("M,K,V", [(16, 768, 50257), (16, 768, 2048), (5, 1536, 300), (1, 776, 129), (3, 200, 17),
                                   (16, 8, 130), (7, 30, 64)])
def test_matmul_t_few_rows_bf16_exact(ctx, M, K, V):
    """x @ w^T with at most 16 rows in the bf16 variant (the LM head of one token per
    sequence, [GPT2-4, "Generation with KV Cache"]): the product of the bf16 operands,
    accumulated in fp32, checked against the float64 product of the rounded operands
    to 1e-5.  k in whole 768-deep passes (768, 1536), with a partial last pass (776,
    200, 8), and not a multiple of 8 (30: the tiled kernel); vocabularies ragged
    against the 128-row workgroups, and one of 50,257 rows whose output rows are
    padded.  The bf16-only output is the exact rounding of the plain one."""
    ctx.set_precision("bf16")
    x, w = rnd(160 + M, (M, K)), rnd(161 + K, (V, K), 1 / np.sqrt(K))
    ts = [ctx.tensor(a.shape, a) for a in (x, w)]
    try:
        y = T.matmul_t(*ts).numpy()
        ref = _bf16_round(x).astype(np.float64) @ _bf16_round(w).astype(np.float64).T
        assert_close(y, ref, 1e-5, "forward")
        ctx.tape_reset()
        yb = T.matmul_t(*ts, bf16_only=True).numpy()
        np.testing.assert_array_equal(yb, _bf16_round(y))
    finally:
        ctx.tape_reset()
        for t in ts:
            t.release()
        ctx.set_precision("fp32")


@pytest.mark.parametrize("case", ["fwd_nn", "bwd_nt"])
def test_linear_one_tile_per_cu(ctx, case):
    """About one 128x192 output tile per CU (768 columns against ~8100 rows, long
    reductions) takes the wide-tile kernel: forward x @ w + b + r (fwd_nn) or the
    backward g @ w^T (bwd_nt), ragged in rows and in the reduction; the tiles at
    the ragged end are checked on their own as well."""
    ctx.set_precision("bf16")
    if case == "fwd_nn":
        arrays = [rnd(131, (8100, 2100)), rnd(132, (2100, 768), 0.02), rnd(133, (768,)), rnd(134, (8100, 768))]
    else:
        arrays = [rnd(135, (8100, 768)), rnd(136, (768, 2304), 0.03), rnd(137, (2304,)), rnd(138, (8100, 2304))]
    R = rnd(139, arrays[3].shape)
    out, grads = gpu_op_with_grads(ctx, lambda x, w, b, r: T.linear(x, w, b, residual=r), arrays, R)
    ref, rgrads = oracle_op_with_grads(lambda x, w, b, r: E.add(r, E.add(E.matmul(x, w), b)), arrays, R)
    ctx.set_precision("fp32")
    assert_close(out, ref, FWD_TOL["bf16"], "forward")
    assert_close(out[-100:], ref[-100:], FWD_TOL["bf16"], "forward, last rows")
    for i, (g, r) in enumerate(zip(grads, rgrads)):
        assert_close(g, r, GRAD_TOL["bf16"], f"grad {i}")
    assert_close(grads[0][-100:], rgrads[0][-100:], GRAD_TOL["bf16"], "dx, last rows")


@pytest.mark.parametrize("case", ["nt_fwd", "nn_fwd", "tn_dw"])
def test_large_products_on_256_tiles(own_ctx, case):
    """Products with at least 512 output tiles of 256x256 in the bf16 variant take
    the kernel that loads its operands straight into LDS: the LM-head shapes, here
    ragged in every dimension.  nt_fwd: x @ w^T with K = 200 (the last k-tile of
    both k-contiguous operands is cleared past K) and 8190 columns (a padded row
    pitch, a partial last group of four); nn_fwd: x @ w with K = 200; tn_dw: the
    weight gradient of x @ w^T, 16300 x 2048 over 520 rows."""
    own_ctx.set_precision("bf16")
    if case == "nt_fwd":
        arrays, build, ob, shape = [rnd(141, (4100, 200)), rnd(142, (8190, 200), 0.1)], T.matmul_t, E.matmul_t, (4100, 8190)
    elif case == "nn_fwd":
        arrays, build, ob, shape = [rnd(143, (4100, 200)), rnd(144, (200, 8192), 0.1)], T.matmul, E.matmul, (4100, 8192)
    else:
        arrays, build, ob, shape = [rnd(145, (520, 2048)), rnd(146, (16300, 2048), 0.02)], T.matmul_t, E.matmul_t, (520, 16300)
    R = rnd(147, shape)
    out, grads = gpu_op_with_grads(own_ctx, build, arrays, R)
    ref, rgrads = oracle_op_with_grads(ob, arrays, R)
    own_ctx.set_precision("fp32")
    assert_close(out, ref, FWD_TOL["bf16"], "forward")
    assert_close(out[-60:, -70:], ref[-60:, -70:], FWD_TOL["bf16"], "forward, last tile corner")
    for i, (g, r) in enumerate(zip(grads, rgrads)):
        assert_close(g, r, GRAD_TOL["bf16"], f"grad {i}")
    assert_close(grads[1][-60:], rgrads[1][-60:], GRAD_TOL["bf16"], "grad 1, last rows")


@pytest.mark.parametrize("case", ["nt_fwd", "nn_fwd", "tn_dw", "tn_split", "nn_split"])
def test_large_products_exact_on_integer_inputs(own_ctx, case):
    """The 256x256-tile products of the test above on integers in [-3, 3]: exact
    in bf16, and every partial sum is an integer below 2**24, so fp32 adds them
    exactly in any order and the results must equal the oracle's bit for bit.  A
    term dropped, repeated or taken from the wrong place anywhere (a tile edge, a
    chunk at an operand's end, a K split) fails, however small its share.
    tn_split: a weight gradient over 8190 rows (760 x 2300), split over K;
    nn_split: the dX of x @ w^T with a 20,000-long reduction, split over K with a
    ragged last k-tile in the last split (and its weight gradient, 20000 x 1540
    over 1030 rows, on whole 256x256 tiles)."""
    rng = np.random.default_rng({"nt_fwd": 151, "nn_fwd": 152, "tn_dw": 153, "tn_split": 154, "nn_split": 155}[case])

    def ints(shape):
        return rng.integers(-3, 4, size=shape).astype(np.float64)

    own_ctx.set_precision("bf16")
    if case == "nt_fwd":
        arrays, build, ob, shape = [ints((4100, 200)), ints((8190, 200))], T.matmul_t, E.matmul_t, (4100, 8190)
    elif case == "nn_fwd":
        arrays, build, ob, shape = [ints((4100, 200)), ints((200, 8192))], T.matmul, E.matmul, (4100, 8192)
    elif case == "tn_dw":
        arrays, build, ob, shape = [ints((520, 2048)), ints((16300, 2048))], T.matmul_t, E.matmul_t, (520, 16300)
    elif case == "tn_split":
        arrays, build, ob, shape = [ints((8190, 760)), ints((760, 2300))], T.matmul, E.matmul, (8190, 2300)
    else:
        arrays, build, ob, shape = [ints((1030, 1540)), ints((20000, 1540))], T.matmul_t, E.matmul_t, (1030, 20000)
    R = ints(shape)
    out, grads = gpu_op_with_grads(own_ctx, build, arrays, R)
    ref, rgrads = oracle_op_with_grads(ob, arrays, R)
    own_ctx.set_precision("fp32")
    bad = np.argwhere(out != ref)
    assert bad.size == 0, f"forward differs at {len(bad)} elements, first {bad[:3].tolist()}"
    for i, (g, r) in enumerate(zip(grads, rgrads)):
        bad = np.argwhere(g != r)
        assert bad.size == 0, f"grad {i} differs at {len(bad)} elements, first {bad[:3].tolist()}"


def test_linear_long_k_split(ctx):
    # a long reduction (the dW contractions of the GPT have K = 8192) takes the split-K path
    check(ctx, "fp32", T.linear, lambda x, w, b: E.add(E.matmul(x, w), b),
          [rnd(8, (4100, 96)), rnd(9, (96, 130), 0.1), rnd(10, (130,))], (4100, 130))


@pytest.mark.parametrize("prec", PRECS)
def test_batch_matmul(ctx, prec):
    check(ctx, prec, T.batch_matmul, E.batch_matmul, [rnd(11, (3, 130, 70)), rnd(12, (3, 70, 150))], (3, 130, 150))


@pytest.mark.parametrize("prec", PRECS)
def test_batch_matmul_t(ctx, prec):
    check(ctx, prec, T.batch_matmul_t, E.batch_matmul_t, [rnd(13, (3, 130, 70)), rnd(14, (3, 150, 70))],
          (3, 130, 150))


def test_add_broadcast_and_same_shape(ctx):
    check(ctx, "fp32", T.add, E.add, [rnd(15, (5, 37, 48)), rnd(16, (48,))], (5, 37, 48))
    check(ctx, "fp32", T.add, E.add, [rnd(17, (5, 37, 47)), rnd(18, (37, 47))], (5, 37, 47))
    check(ctx, "fp32", T.add, E.add, [rnd(19, (300, 257)), rnd(20, (300, 257))], (300, 257))


@pytest.mark.parametrize("name", ["mul", "scale", "tanh", "gelu", "reshape", "sum"])
def test_pointwise(ctx, name):
    a, b = rnd(21, (300, 257), 2.0), rnd(22, (300, 257))
    if name == "mul":
        check(ctx, "fp32", T.mul, E.mul, [a, b], a.shape)
    elif name == "scale":
        check(ctx, "fp32", lambda x: T.scale(x, 0.37), lambda x: E.scale(x, 0.37), [a], a.shape)
    elif name == "tanh":
        check(ctx, "fp32", T.tanh, E.tanh, [a], a.shape)
    elif name == "gelu":
        check(ctx, "fp32", T.gelu, E.gelu, [a], a.shape)
    elif name == "reshape":
        check(ctx, "fp32", lambda x: T.reshape(x, (257, 300)), lambda x: E.reshape(x, (257, 300)), [a], (257, 300))
    else:
        check(ctx, "fp32", T.sum_all, E.sum_all, [a], (1,))


@pytest.mark.parametrize("C", [768, 100, 400, 1000, 1500])
def test_layernorm(ctx, C):
    """Row widths of 1, 3 (partly filled: 400), 3 (exactly: 768) and 4 (1000) float4s per
    lane in the fused backward, and one (1500) past it."""
    x = rnd(23, (3, 70, C), 2.0) + 0.5
    g, b = 1 + rnd(24, (C,), 0.2), rnd(25, (C,), 0.2)
    check(ctx, "fp32", lambda x, g, b: T.layernorm(x, g, b, 1e-5), lambda x, g, b: E.layernorm(x, g, b, 1e-5),
          [x, g, b], x.shape)


def test_layernorm_more_rows_than_one_pass(ctx):
    """8400 rows of 768: more than the fused backward's workgroups take in one pass
    of two rows per wave, so some waves take a second pass with a single row."""
    x = rnd(28, (2, 4200, 768), 2.0) + 0.5
    g, b = 1 + rnd(29, (768,), 0.2), rnd(30, (768,), 0.2)
    check(ctx, "fp32", lambda x, g, b: T.layernorm(x, g, b, 1e-5), lambda x, g, b: E.layernorm(x, g, b, 1e-5),
          [x, g, b], x.shape)


def test_embedding(ctx):
    table = rnd(26, (50, 40))
    ids = S.random_ids(27, (6, 35), 50)
    check(ctx, "fp32", lambda t: T.embedding(t, ids, 6), lambda t: E.embedding(t, ids.reshape(-1), 6), [table],
          (6, 35, 40))


def test_embedding_routing_is_bit_exact(ctx):
    """Forward rows are bitwise the table rows; with integer upstream gradients the
    scatter-add sums are exact in fp32, so the table gradient must equal the
    oracle's hit counts bit for bit (more ids than one sort chunk)."""
    V, C, n = 97, 33, 9000
    table = rnd(28, (V, C))
    ids = S.random_ids(29, (n,), V)
    up = S.rng_for(30).integers(-3, 4, size=(1, n, C)).astype(np.float32)
    t = ctx.tensor(table.shape, table)
    out = T.embedding(t, ids, 1)
    assert np.array_equal(out.numpy().reshape(n, C), table[ids])
    Rt = ctx.tensor(up.shape, up)
    ctx.backward(T.sum_all(T.mul(out, Rt)))
    expect = np.zeros((V, C), np.float64)
    np.add.at(expect, ids, up.reshape(n, C))
    assert np.array_equal(t.grad(), expect.astype(np.float32))
    ctx.tape_reset()
    t.release()
    Rt.release()


@pytest.mark.parametrize("reps", [[1, 62, 63, 64, 65, 1], [1300, 2, 700, 127, 128, 129]])
def test_embedding_backward_long_runs_exact(ctx, reps):
    """[Autograd-1, table of ops: Embedding] backward: a wave reads a window of 64
    sorted keys at once, so runs of equal ids of 62..65 (the window's edge) and runs
    far longer than a window (the rest of the run read key by key) must still sum
    every row once; integer gradients make the sums exact, so the check is bit for bit
    (the ids are shuffled, so the sort builds the runs; 2,386 ids fit one chunk)."""
    C = 70
    base = np.concatenate([np.full(r, i, np.int32) for i, r in enumerate(reps)])
    ids = base[S.rng_for(31).permutation(base.size)]
    n, V = ids.size, len(reps)
    table = rnd(32, (V, C))
    up = S.rng_for(33).integers(-3, 4, size=(1, n, C)).astype(np.float32)
    t = ctx.tensor(table.shape, table)
    Rt = ctx.tensor(up.shape, up)
    try:
        out = T.embedding(t, ids, 1)
        ctx.backward(T.sum_all(T.mul(out, Rt)))
        expect = np.zeros((V, C), np.float64)
        np.add.at(expect, ids, up.reshape(n, C))
        assert np.array_equal(t.grad(), expect.astype(np.float32))
    finally:
        ctx.tape_reset()
        t.release()
        Rt.release()


def test_narrow_split_merge(ctx):
    x = rnd(31, (2, 37, 3 * 96))
    check(ctx, "fp32", lambda a: T.narrow(a, 96, 96), lambda a: E.narrow(a, 96, 96), [x], (2, 37, 96))
    y = rnd(32, (2, 37, 96))
    check(ctx, "fp32", lambda a: T.split_heads(a, 3), lambda a: E.split_heads(a, 3), [y], (2, 3, 37, 32))
    z = rnd(33, (2, 3, 37, 32))
    check(ctx, "fp32", T.merge_heads, E.merge_heads, [z], (2, 37, 96))


def test_causal_softmax(ctx):
    s = rnd(34, (2, 3, 130, 130), 3.0)
    check(ctx, "fp32", T.causal_softmax, E.causal_softmax, [s], s.shape)


def _attention_oracle(qkv, heads):
    B, Tn, C3 = qkv.shape
    C = C3 // 3
    hs = C // heads
    q = E.split_heads(E.narrow(qkv, 0, C), heads)
    k = E.split_heads(E.narrow(qkv, C, C), heads)
    v = E.split_heads(E.narrow(qkv, 2 * C, C), heads)
    r = lambda t: E.reshape(t, (B * heads, Tn, hs))
    p = E.causal_softmax(E.scale(E.batch_matmul_t(r(q), r(k)), 1.0 / math.sqrt(hs)))
    return E.merge_heads(E.reshape(E.batch_matmul(p, r(v)), (B, heads, Tn, hs)))


@pytest.mark.parametrize("prec", PRECS)
@pytest.mark.parametrize("B,Tn,H,hs", [(2, 200, 3, 32), (2, 130, 2, 64), (1, 1, 2, 64), (3, 64, 4, 32)])
def test_causal_attention_equals_op_composition(ctx, prec, B, Tn, H, hs):
    qkv = rnd(35, (B, Tn, 3 * H * hs))
    check(ctx, prec, lambda a: T.causal_attention(a, H), lambda a: _attention_oracle(a, H), [qkv],
          (B, Tn, H * hs))


def test_attention_composed_from_ops_on_gpu(ctx):
    """The separate GPU ops (Narrow/SplitHeads/BatchMatMulT/Scale/CausalSoftmax/
    BatchMatMul/MergeHeads) give the same result as the oracle composition."""
    B, Tn, H, hs = 2, 70, 2, 32
    C = H * hs

    def gpu(a):
        q = T.split_heads(T.narrow(a, 0, C), H)
        k = T.split_heads(T.narrow(a, C, C), H)
        v = T.split_heads(T.narrow(a, 2 * C, C), H)
        r = lambda t: T.reshape(t, (B * H, Tn, hs))
        p = T.causal_softmax(T.scale(T.batch_matmul_t(r(q), r(k)), 1.0 / math.sqrt(hs)))
        return T.merge_heads(T.reshape(T.batch_matmul(p, r(v)), (B, H, Tn, hs)))
    check(ctx, "fp32", gpu, lambda a: _attention_oracle(a, H), [rnd(36, (B, Tn, 3 * C))], (B, Tn, C))


@pytest.mark.parametrize("rows,V", [(300, 1000), (37, 50257)])
def test_softmax_cross_entropy(ctx, rows, V):
    logits = rnd(37, (rows, V), 3.0)
    tg = S.random_ids(38, (rows,), V)
    ctx.set_precision("fp32")
    lt = ctx.tensor(logits.shape, logits)
    loss = T.softmax_cross_entropy(lt, tg)
    ctx.backward(loss)
    ref = E.Tensor(logits.astype(np.float64))
    rl = E.softmax_cross_entropy(ref, tg)
    rl.backward()
    assert abs(loss.item() - rl.item()) / max(abs(rl.item()), 1) <= 1e-5
    assert_close(lt.grad(), ref.grad, 1e-4, "dlogits")
    ctx.tape_reset()
    lt.release()


def test_ce_uniform_logits_is_log_v(ctx):
    V = 50257
    lt = ctx.tensor((4, V), np.zeros((4, V), np.float32))
    loss = T.softmax_cross_entropy(lt, np.array([0, 1, V - 1, 7]))
    assert abs(loss.item() - math.log(V)) < 1e-5
    ctx.tape_reset()
    lt.release()


# ----------------------------------------------------------------------------- tape semantics
def test_tensor_used_twice_accumulates(ctx):
    """[Autograd-1, "Why += and not ="]: L = z*z at z = 7 gives dL/dz = 14."""
    z = ctx.tensor((1,), [7.0])
    ctx.backward(T.mul(z, z))
    assert z.grad()[0] == 14.0
    ctx.tape_reset()
    z.release()


def test_tiny_graph_values(ctx):
    w, x, b = (ctx.tensor((1,), [v]) for v in (2.0, 3.0, 1.0))
    z = T.add(T.mul(w, x), b)
    L = T.mul(z, z)
    ctx.backward(L)
    assert (z.item(), L.item()) == (7.0, 49.0)
    assert (z.grad()[0], w.grad()[0], x.grad()[0], b.grad()[0]) == (14.0, 42.0, 28.0, 14.0)
    ctx.tape_reset()
    for t in (w, x, b):
        t.release()


def test_leaf_grads_accumulate_until_zero_grad(ctx):
    w = ctx.tensor((4,), [1, 2, 3, 4])
    x = ctx.tensor((4,), [5, 6, 7, 8])
    for k in (1, 2):
        ctx.backward(T.sum_all(T.mul(w, x)))
        assert np.array_equal(w.grad(), k * np.array([5, 6, 7, 8], np.float32))
    ctx.zero_grad([w])
    assert np.array_equal(w.grad(), np.zeros(4, np.float32))
    ctx.backward(T.sum_all(T.mul(w, x)))
    assert np.array_equal(w.grad(), np.array([5, 6, 7, 8], np.float32))
    ctx.tape_reset()
    w.release()
    x.release()


def test_errors_are_reported_and_context_survives(ctx):
    a = ctx.tensor((3, 4))
    b = ctx.tensor((5, 6))
    with pytest.raises(T.TfbError) as e:
        T.matmul(a, b)
    assert e.value.code == -2
    with pytest.raises(T.TfbError):
        T.mul(a, b)
    y = T.tanh(a)
    with pytest.raises(T.TfbError) as e:
        ctx.backward(y)
    assert e.value.code == -3 and "scalar" in str(e.value)
    with pytest.raises(T.TfbError):
        T.softmax_cross_entropy(a, np.zeros(2, np.int32))
    # still usable
    ctx.backward(T.sum_all(T.tanh(a)))
    assert np.allclose(a.grad(), 1.0)
    ctx.tape_reset()
    a.release()
    b.release()


def test_add_of_single_use_outputs_and_repeated_backward(ctx):
    """[Autograd-1, "Backward pass"]: an op output read only by an Add gets exactly the
    Add's output gradient (the library lets it use that buffer), leaf gradients add up
    over repeated backward passes, and intermediate gradients are per pass."""
    xv, zv, rv = rnd(41, (6, 40)), rnd(42, (6, 40)), rnd(43, (6, 40))
    x = ctx.tensor(xv.shape, xv)
    z = ctx.tensor(zv.shape, zv)
    R = ctx.tensor(rv.shape, rv)
    p, q = T.tanh(x), T.gelu(z)                  # each read once, by the Add
    s_ = T.add(p, q)
    loss = T.sum_all(T.mul(s_, R))
    ctx.backward(loss)
    ctx.backward(loss)                           # a second pass over the same tape
    X, Z = E.Tensor(xv.astype(np.float64)), E.Tensor(zv.astype(np.float64))
    P, Q = E.tanh(X), E.gelu(Z)
    L = E.sum_all(E.mul(E.add(P, Q), E.Tensor(rv.astype(np.float64))))
    L.backward()
    assert_close(p.grad(), rv, 1e-6, "p.grad")
    assert_close(q.grad(), rv, 1e-6, "q.grad")
    assert_close(s_.grad(), rv, 1e-6, "s.grad")
    assert_close(x.grad(), 2 * X.grad, 1e-5, "x.grad after two passes")
    assert_close(z.grad(), 2 * Z.grad, 1e-5, "z.grad after two passes")
    ctx.tape_reset()
    for t in (x, z, R):
        t.release()


@pytest.mark.parametrize("prec", PRECS)
def test_residual_gradients_without_copies(ctx, prec):
    """[Autograd-1, "Backward pass"]: gradients of residual-stream tensors, which the
    library carries from an Add to the tensor's next contribution without a copy:
    taken up by a LayerNorm backward (x0), by another op's contribution (u, read by a
    Mul recorded before the Add), or by no further op at all (v: its other reader
    does not reach the loss).  Two passes over one tape; leaf gradients add up."""
    ctx.set_precision(prec)
    xin, uin, vin = rnd(81, (4, 24, 64)), rnd(82, (4, 24, 64)), rnd(83, (4, 24, 64))
    gam, bet = rnd(84, (64,), 0.5) + 1.0, rnd(85, (64,), 0.1)
    Wv, bv, Rv, Mv = rnd(86, (64, 64), 0.1), rnd(87, (64,), 0.1), rnd(88, (4, 24, 64)), rnd(89, (4, 24, 64))
    leaves = {k: ctx.tensor(v.shape, v) for k, v in
              dict(xin=xin, uin=uin, vin=vin, gam=gam, bet=bet, W=Wv, b=bv, R=Rv, M=Mv).items()}
    L = leaves

    def build(ops, t):
        x0 = ops.tanh(t["xin"])
        y = ops.add(ops.matmul(ops.layernorm(x0, t["gam"], t["bet"]), t["W"]), t["b"])
        x1 = ops.add(x0, y)                                  # x0: deferred, then the LayerNorm's share
        u = ops.tanh(t["uin"])
        m = ops.mul(u, t["M"])                               # u's other reader, recorded before the Add
        x2 = ops.add(u, ops.gelu(x1))                        # u: deferred, then the Mul's share
        v = ops.tanh(t["vin"])
        ops.gelu(v)                                          # v's other reader: not on the loss path
        x3 = ops.add(v, ops.mul(x2, m))                      # v: deferred, nothing else arrives
        return ops.sum_all(ops.mul(x3, t["R"])), (x0, u, v)

    loss, inter = build(T, L)
    ctx.backward(loss)
    ctx.backward(loss)
    O = {k: E.Tensor(a.astype(np.float64)) for k, a in
         dict(xin=xin, uin=uin, vin=vin, gam=gam, bet=bet, W=Wv, b=bv, R=Rv, M=Mv).items()}
    oloss, ointer = build(E, O)
    oloss.backward()
    tol = GRAD_TOL[prec]
    for name, g, r in zip(("x0", "u", "v"), inter, ointer):
        assert_close(g.grad(), r.grad, tol, f"{name}.grad (one pass)")
    for k in ("xin", "uin", "vin", "gam", "bet", "W", "b", "M"):
        assert_close(L[k].grad(), 2 * O[k].grad, tol, f"{k}.grad after two passes")
    ctx.tape_reset()
    for t in L.values():
        t.release()
    ctx.set_precision("fp32")


def test_linear_bf16_copy_changes_nothing(ctx):
    """The bf16 copy a linear's product writes for its reader (here the attention
    kernels) is the same rounding the reader would have made: outputs and every
    gradient agree bit for bit with the plain linear."""
    ctx.set_precision("bf16")
    B, Tn, C, H = 2, 96, 128, 2
    xv, wv, bv, rv = rnd(91, (B, Tn, C)), rnd(92, (C, 3 * C), 0.05), rnd(93, (3 * C,), 0.1), rnd(94, (B, Tn, C))
    res = []
    for flag in (False, True):
        x, w, b, R = (ctx.tensor(a.shape, a) for a in (xv, wv, bv, rv))
        y = T.causal_attention(T.linear(x, w, b, bf16_copy=flag), H)
        ctx.backward(T.sum_all(T.mul(y, R)))
        res.append([y.numpy(), x.grad(), w.grad(), b.grad()])
        ctx.tape_reset()
        for t in (x, w, b, R):
            t.release()
    for a, b_ in zip(*res):
        np.testing.assert_array_equal(a, b_)
    ctx.set_precision("fp32")


@pytest.mark.parametrize("grad_only", [False, True])
def test_cross_entropy_of_bf16_only_logits(ctx, grad_only):
    """Logits stored as bf16 alone (an LM head with the bf16-only output flag, rows
    padded past 1030 columns) are exactly the bf16 rounding of the plain product; the
    cross-entropy reads them directly: its loss is the oracle's on those bf16 values,
    and the gradients (upstream gradient 1, then 3) stay within the bf16 tolerance."""
    V, C, rows = 1030, 64, 300
    x, w = rnd(47, (rows, C)), rnd(48, (V, C), 0.2)
    tg = S.random_ids(49, (rows,), V)
    ctx.set_precision("bf16")
    xt, wt = ctx.tensor(x.shape, x), ctx.tensor(w.shape, w)
    plain = T.matmul_t(xt, wt).numpy()
    ctx.tape_reset()
    for up in (1.0, 3.0):
        logits = T.matmul_t(xt, wt, bf16_only=True)
        got = logits.numpy()
        np.testing.assert_array_equal(got, _bf16_round(plain))
        loss = T.softmax_cross_entropy(logits, tg, bf16_grad_only=grad_only)
        ctx.backward(T.scale(loss, up))
        lv, dx, dw = loss.numpy(), xt.grad(), wt.grad()
        if grad_only:
            with pytest.raises(T.TfbError):
                logits.grad()
        ctx.tape_reset()
        want = E.softmax_cross_entropy(E.Tensor(got.astype(np.float64)), tg).data
        assert_close(lv, want, 1e-5, f"loss (upstream {up})")
        ox, ow = E.Tensor(x.astype(np.float64)), E.Tensor(w.astype(np.float64))
        E.scale(E.softmax_cross_entropy(E.matmul_t(ox, ow), tg), up).backward()
        assert_close(dx, ox.grad, GRAD_TOL["bf16"], f"dx (upstream {up})")
        assert_close(dw, ow.grad, GRAD_TOL["bf16"], f"dw (upstream {up})")
        ctx.zero_grad([xt, wt])   # leaf gradients add up over backward passes
    xt.release()
    wt.release()
    ctx.set_precision("fp32")


@pytest.mark.parametrize("prec", PRECS)
def test_cross_entropy_bf16_only_logit_gradient(ctx, prec):
    """With the bf16-only option, an LM head's gradients are those of the plain call
    (up to the last bit of the log-sum-exp in the bf16 variant, where the forward also
    writes the gradient), and the option is ignored in fp32.  The logits' own fp32 gradient is not kept (bf16 only);
    logits with another reader keep the plain behaviour."""
    V, C, rows = 1030, 64, 300
    x, w = rnd(44, (rows, C)), rnd(45, (V, C), 0.2)
    tg = S.random_ids(46, (rows,), V)
    ctx.set_precision(prec)
    res = []
    for only in (False, True):
        xt, wt = ctx.tensor(x.shape, x), ctx.tensor(w.shape, w)
        logits = T.matmul_t(xt, wt)
        loss = T.softmax_cross_entropy(logits, tg, bf16_grad_only=only)
        ctx.backward(loss)
        ctx.backward(loss)                                   # a second pass: leaf gradients add up
        res.append([loss.numpy(), xt.grad(), wt.grad()])
        if only and prec == "bf16":
            with pytest.raises(T.TfbError):
                logits.grad()
        else:
            res[-1].append(logits.grad())
        ctx.tape_reset()
        xt.release()
        wt.release()
    # in the bf16 variant the option also takes the gradient from the forward's single
    # pass over the logits (max, then sum: the log-sum-exp may differ in its last bit)
    tols = [1e-6, 1e-3, 1e-3, 1e-6] if prec == "bf16" else [0, 0, 0, 0]
    for a, b_, tol in zip(res[0], res[1], tols):
        if tol == 0:
            np.testing.assert_array_equal(a, b_)
        else:
            assert_close(a, b_, tol, "bf16-only against plain")
    # an upstream gradient other than 1: the backward recomputes (scaled) gradients
    xt, wt = ctx.tensor(x.shape, x), ctx.tensor(w.shape, w)
    loss = T.scale(T.softmax_cross_entropy(T.matmul_t(xt, wt), tg, bf16_grad_only=True), 3.0)
    ctx.backward(loss)
    ox, ow = E.Tensor(x.astype(np.float64)), E.Tensor(w.astype(np.float64))
    E.scale(E.softmax_cross_entropy(E.matmul_t(ox, ow), tg), 3.0).backward()
    assert_close(xt.grad(), ox.grad, GRAD_TOL[prec], "dx, upstream gradient 3")
    assert_close(wt.grad(), ow.grad, GRAD_TOL[prec], "dw, upstream gradient 3")
    ctx.tape_reset()
    xt.release()
    wt.release()
    # another reader of the logits: the option does not apply
    xt, wt = ctx.tensor(x.shape, x), ctx.tensor(w.shape, w)
    logits = T.matmul_t(xt, wt)
    loss = T.add(T.softmax_cross_entropy(logits, tg, bf16_grad_only=True), T.sum_all(T.scale(logits, 1e-3)))
    ctx.backward(loss)
    assert np.isfinite(logits.grad()).all()
    ctx.tape_reset()
    xt.release()
    wt.release()
    ctx.set_precision("fp32")


@pytest.mark.parametrize("prec", PRECS)
def test_bias_gradients_from_fused_column_sums(ctx, prec):
    """[Autograd-1, "Backward pass"; "Ops": the bias Add's rule sums g over rows]: a
    Linear's bias gradient taken from the column sums that the kernel finishing its
    output gradient leaves behind -- a LayerNorm backward (residual stream) and a GELU
    backward (the MLP) -- against the oracle.  1000 and 300 rows: several row slabs
    with ragged ends."""
    ctx.set_precision(prec)
    for rows in (1000, 300):
        xin, R = rnd(101, (rows, 64)), rnd(102, (rows, 128))
        gam, bet = rnd(103, (64,), 0.5) + 1.0, rnd(104, (64,), 0.1)
        W1, b1 = rnd(105, (64, 128), 0.1), rnd(106, (128,), 0.1)
        W2, b2 = rnd(107, (128, 64), 0.1), rnd(108, (64,), 0.1)
        gam2, bet2 = rnd(109, (64,), 0.5) + 1.0, rnd(110, (64,), 0.1)
        arrs = dict(xin=xin, gam=gam, bet=bet, W1=W1, b1=b1, W2=W2, b2=b2, gam2=gam2, bet2=bet2, R=R)

        def gpu(t):
            x0 = T.tanh(t["xin"])
            h = T.linear(T.layernorm(x0, t["gam"], t["bet"]), t["W1"], t["b1"])
            a = T.gelu(h)                                     # b1: from the GELU backward's sums
            x1 = T.add(x0, T.linear(a, t["W2"], t["b2"]))      # b2: from the LayerNorm backward's sums
            y = T.layernorm(x1, t["gam2"], t["bet2"])
            return T.sum_all(T.mul(T.linear(y, t["W1"], t["b1"]), t["R"]))

        def ora(t):
            x0 = E.tanh(t["xin"])
            h = E.add(E.matmul(E.layernorm(x0, t["gam"], t["bet"]), t["W1"]), t["b1"])
            x1 = E.add(x0, E.add(E.matmul(E.gelu(h), t["W2"]), t["b2"]))
            y = E.layernorm(x1, t["gam2"], t["bet2"])
            return E.sum_all(E.mul(E.add(E.matmul(y, t["W1"]), t["b1"]), t["R"]))

        G = {k: ctx.tensor(v.shape, v) for k, v in arrs.items()}
        ctx.backward(gpu(G))
        O = {k: E.Tensor(v.astype(np.float64)) for k, v in arrs.items()}
        ora(O).backward()
        for k in ("b1", "b2", "W1", "W2", "xin", "gam", "bet"):
            assert_close(G[k].grad(), O[k].grad, GRAD_TOL[prec], f"{k}.grad ({rows} rows)")
        ctx.tape_reset()
        for t in G.values():
            t.release()
    ctx.set_precision("fp32")


@pytest.mark.parametrize("prec", PRECS)
def test_bf16_only_outputs(ctx, prec):
    """Outputs kept as bf16 copies alone (LayerNorm, GELU, Linear): read back as the exact
    bf16 rounding of the plain op's output (unchanged in fp32); a contraction or attention
    reading them and every gradient are bit-identical to the plain ops, except qkv's bias
    gradient in the bf16 variant: its gradient is then kept as bf16 alone, so that bias
    gradient is the column sum of those bf16 values; an fp32 reader (Tanh) sees the
    converted values."""
    ctx.set_precision(prec)
    B, Tn, C, H = 2, 80, 64, 2
    xv, g1, b1 = rnd(131, (B, Tn, C)), rnd(132, (C,), 0.5) + 1.0, rnd(133, (C,), 0.1)
    W1, c1 = rnd(134, (C, 3 * C), 0.1), rnd(135, (3 * C,), 0.1)
    W2, c2 = rnd(136, (C, 96), 0.1), rnd(137, (96,), 0.1)
    R1, R2 = rnd(138, (B, Tn, C)), rnd(139, (B, Tn, 96))
    res = []
    for only in (False, True):
        t = {k: ctx.tensor(v.shape, v) for k, v in dict(x=xv, g1=g1, b1=b1, W1=W1, c1=c1, W2=W2, c2=c2,
                                                          R1=R1, R2=R2).items()}
        h = T.layernorm(t["x"], t["g1"], t["b1"], bf16_only=only)
        qkv = T.linear(h, t["W1"], t["c1"], bf16_only=only)
        att = T.causal_attention(qkv, H)
        f = T.gelu(T.linear(h, t["W2"], t["c2"]), bf16_only=only)
        th = T.tanh(f)                                            # an fp32 reader
        loss = T.add(T.sum_all(T.mul(att, t["R1"])), T.sum_all(T.mul(th, t["R2"])))
        ctx.backward(loss)
        res.append(dict(h=h.numpy(), qkv=qkv.numpy(), f=f.numpy(), att=att.numpy(), th=th.numpy(),
                        **{"d" + k: t[k].grad() for k in ("x", "g1", "b1", "W1", "c1", "W2", "c2")}))
        if not only:
            res[-1]["dqkv"] = qkv.grad()
        ctx.tape_reset()
        for v in t.values():
            v.release()
    plain, only = res
    for k in ("h", "qkv", "f"):
        want = _bf16_round(plain[k]) if prec == "bf16" else plain[k]
        np.testing.assert_array_equal(only[k], want, err_msg=k)
    np.testing.assert_array_equal(only["att"], plain["att"])
    # Tanh reads the converted bf16 values (exactly those) in the bf16 variant
    assert_close(only["th"], np.tanh(only["f"].astype(np.float64)), 1e-6, "tanh of the bf16-only output")
    if prec == "fp32":
        np.testing.assert_array_equal(only["th"], plain["th"])
    np.testing.assert_array_equal(only["dW1"], plain["dW1"], err_msg="dW1")  # the contraction reads bf16 in both
    if prec == "fp32":
        np.testing.assert_array_equal(only["dc1"], plain["dc1"], err_msg="dc1")
    else:
        want = _bf16_round(plain["dqkv"]).astype(np.float64).reshape(-1, 3 * C).sum(axis=0)
        assert_close(only["dc1"], want, 1e-5, "dc1: column sums of the bf16 gradient")
    for k in ("dx", "dg1", "db1", "dW2", "dc2"):               # the Tanh branch sees rounded inputs
        assert_close(only[k], plain[k], 1e-6 if prec == "fp32" else 2e-2, k)
    ctx.set_precision("fp32")


def test_gelu_of_bf16_only_input(ctx):
    """A GELU whose input (a Linear's output) is held only as bf16 reads those bf16 values:
    its output is exactly the plain GELU of the bf16-rounded product, and its gradients
    stay within the bf16 tolerance of the oracle (300 and 1000 rows: the row-slab
    backward and its ragged end).  The product's gradient is then written only as the
    bf16 copy its backward reads, so reading it is an error."""
    ctx.set_precision("bf16")
    for rows in (300, 1000):
        xv, W, bv, Rv = rnd(141, (rows, 64)), rnd(142, (64, 96), 0.2), rnd(143, (96,), 0.1), rnd(144, (rows, 96))
        x, w, b, R = (ctx.tensor(a.shape, a) for a in (xv, W, bv, Rv))
        lin_plain = T.linear(x, w, b).numpy()
        ctx.tape_reset()
        lin = T.linear(x, w, b, bf16_only=True)
        f = T.gelu(lin, bf16_only=True)
        ctx.backward(T.sum_all(T.mul(T.tanh(f), R)))
        got = f.numpy()
        dx, dw, db = x.grad(), w.grad(), b.grad()
        with pytest.raises(T.TfbError):   # the product's gradient was kept only as bf16
            lin.grad()
        ctx.tape_reset()
        rin = ctx.tensor(lin_plain.shape, _bf16_round(lin_plain))
        want = _bf16_round(T.gelu(rin).numpy())
        ctx.tape_reset()
        np.testing.assert_array_equal(got, want)
        ox, ow, ob = (E.Tensor(a.astype(np.float64)) for a in (xv, W, bv))
        E.sum_all(E.mul(E.tanh(E.gelu(E.add(E.matmul(ox, ow), ob))), E.Tensor(Rv.astype(np.float64)))).backward()
        for g_, o_, name in ((dx, ox.grad, "dx"), (dw, ow.grad, "dw"), (db, ob.grad, "db")):
            assert_close(g_, o_, GRAD_TOL["bf16"], f"{name} ({rows} rows)")
        for t in (x, w, b, R, rin):
            t.release()
    ctx.set_precision("fp32")


def test_mlp_gelu_gradient_kept_as_bf16(ctx):
    """An MLP block as the GPT runs it: Linear (bf16-only output) -> GELU (bf16-only
    output) -> Linear.  The second Linear's dX is then written as bf16 alone and the
    GELU backward reads it that way (reading the GELU output's gradient is an error);
    every parameter gradient stays within the bf16 tolerance of the oracle (300 rows:
    the row-slab backward and its ragged end)."""
    ctx.set_precision("bf16")
    xv, W1, b1, W2, b2 = rnd(151, (300, 64)), rnd(152, (64, 96), 0.2), rnd(153, (96,), 0.1), rnd(154, (96, 40), 0.2), \
        rnd(155, (40,), 0.1)
    R = rnd(156, (300, 40))
    ts = [ctx.tensor(a.shape, a) for a in (xv, W1, b1, W2, b2)]
    x, w1, bb1, w2, bb2 = ts
    f = T.gelu(T.linear(x, w1, bb1, bf16_only=True), bf16_only=True)
    y = T.linear(f, w2, bb2)
    Rt = ctx.tensor(R.shape, R)
    ctx.backward(T.sum_all(T.mul(y, Rt)))
    grads = [t.grad() for t in ts]
    with pytest.raises(T.TfbError):
        f.grad()
    ctx.tape_reset()
    for t in ts + [Rt]:
        t.release()
    ctx.set_precision("fp32")
    os_ = [E.Tensor(a.astype(np.float64)) for a in (xv, W1, b1, W2, b2)]
    ox, ow1, ob1, ow2, ob2 = os_
    E.sum_all(E.mul(E.add(E.matmul(E.gelu(E.add(E.matmul(ox, ow1), ob1)), ow2), ob2),
                    E.Tensor(R.astype(np.float64)))).backward()
    for g_, o_, name in zip(grads, os_, ("dx", "dw1", "db1", "dw2", "db2")):
        assert_close(g_, o_.grad, GRAD_TOL["bf16"], name)


@pytest.mark.parametrize("out_only", [False, True])
def test_attention_qkv_gradient_kept_as_bf16(ctx, out_only):
    """qkv from a Linear with the bf16-only output flag, then the fused attention: its
    backward writes the qkv gradient as bf16 alone, the Linear reads it (and sums its
    columns for the bias gradient) as such, and reading qkv's gradient is an error.
    out_only: the attention output is bf16-only too and feeds a projection, whose dX
    is then written as bf16 alone (the backward takes rowsum(dy * y) from the bf16
    copies).  Gradients of every input against the oracle (ragged T = 130, 2 heads of 32)."""
    ctx.set_precision("bf16")
    B, Tn, C, H = 2, 130, 64, 2
    xv, W, bv = rnd(161, (B, Tn, C)), rnd(162, (C, 3 * C), 0.2), rnd(163, (3 * C,), 0.1)
    Wp, bp = rnd(165, (C, C), 0.2), rnd(166, (C,), 0.1)
    R = rnd(164, (B, Tn, C))
    ts = [ctx.tensor(a.shape, a) for a in (xv, W, bv, Wp, bp)]
    qkv = T.linear(ts[0], ts[1], ts[2], bf16_only=True)
    y = T.causal_attention(qkv, H, bf16_only=out_only)
    y = T.linear(y, ts[3], ts[4])
    Rt = ctx.tensor(R.shape, R)
    ctx.backward(T.sum_all(T.mul(y, Rt)))
    grads = [t.grad() for t in ts]
    with pytest.raises(T.TfbError):
        qkv.grad()
    ctx.tape_reset()
    for t in ts + [Rt]:
        t.release()
    ctx.set_precision("fp32")
    os_ = [E.Tensor(a.astype(np.float64)) for a in (xv, W, bv, Wp, bp)]
    oq = E.add(E.matmul(os_[0], os_[1]), os_[2])
    oy = E.add(E.matmul(_attention_oracle(oq, H), os_[3]), os_[4])
    E.sum_all(E.mul(oy, E.Tensor(R.astype(np.float64)))).backward()
    for g_, o_, name in zip(grads, os_, ("dx", "dw", "db", "dwp", "dbp")):
        assert_close(g_, o_.grad, GRAD_TOL["bf16"], name)


@pytest.mark.parametrize("C", [64, 768])
def test_layernorm_gradient_kept_as_bf16(ctx, C):
    """LayerNorm with the bf16-only output flag feeding a Linear: the Linear's dX is
    written as bf16 alone and the fused LayerNorm backward reads it that way (reading
    the LayerNorm output's gradient is an error).  Every input's gradient against the
    oracle (300 rows, C = 64 and the GPT's 768)."""
    ctx.set_precision("bf16")
    xv, gv, bv = rnd(171, (300, C), 2.0) + 0.5, 1 + rnd(172, (C,), 0.2), rnd(173, (C,), 0.2)
    W, c = rnd(174, (C, 40), 0.2), rnd(175, (40,), 0.1)
    R = rnd(176, (300, 40))
    ts = [ctx.tensor(a.shape, a) for a in (xv, gv, bv, W, c)]
    h = T.layernorm(ts[0], ts[1], ts[2], bf16_only=True)
    y = T.linear(h, ts[3], ts[4])
    Rt = ctx.tensor(R.shape, R)
    ctx.backward(T.sum_all(T.mul(y, Rt)))
    grads = [t.grad() for t in ts]
    with pytest.raises(T.TfbError):
        h.grad()
    ctx.tape_reset()
    for t in ts + [Rt]:
        t.release()
    ctx.set_precision("fp32")
    os_ = [E.Tensor(a.astype(np.float64)) for a in (xv, gv, bv, W, c)]
    oy = E.add(E.matmul(E.layernorm(os_[0], os_[1], os_[2], 1e-5), os_[3]), os_[4])
    E.sum_all(E.mul(oy, E.Tensor(R.astype(np.float64)))).backward()
    for g_, o_, name in zip(grads, os_, ("dx", "dgamma", "dbeta", "dw", "db")):
        assert_close(g_, o_.grad, GRAD_TOL["bf16"], name)


@pytest.mark.parametrize("prec", PRECS)
def test_shared_parameters_accumulate_through_deferred_sums(ctx, prec):
    """One LayerNorm's gamma/beta and one Linear's weight/bias used twice in a row
    (x -> LN -> Linear -> GELU -> LN -> Linear): the bias and LayerNorm gradients come
    from column sums that are queued and run at the end of the backward pass; the second
    contribution to each shared gradient must land on the first.  Every gradient against
    the oracle (300 rows, 64 columns)."""
    ctx.set_precision(prec)
    C = 64
    xv, gv, bv = rnd(181, (300, C), 2.0), 1 + rnd(182, (C,), 0.2), rnd(183, (C,), 0.2)
    W, c = rnd(184, (C, C), 0.2), rnd(185, (C,), 0.1)
    R = rnd(186, (300, C))
    ts = [ctx.tensor(a.shape, a) for a in (xv, gv, bv, W, c)]
    x, g, b, w, cb = ts
    h = T.linear(T.layernorm(x, g, b), w, cb)
    y = T.linear(T.layernorm(T.gelu(h), g, b), w, cb)
    Rt = ctx.tensor(R.shape, R)
    ctx.backward(T.sum_all(T.mul(y, Rt)))
    grads = [t.grad() for t in ts]
    ctx.tape_reset()
    for t in ts + [Rt]:
        t.release()
    ctx.set_precision("fp32")
    os_ = [E.Tensor(a.astype(np.float64)) for a in (xv, gv, bv, W, c)]
    ox, og, ob, ow, oc = os_
    oh = E.add(E.matmul(E.layernorm(ox, og, ob, 1e-5), ow), oc)
    oy = E.add(E.matmul(E.layernorm(E.gelu(oh), og, ob, 1e-5), ow), oc)
    E.sum_all(E.mul(oy, E.Tensor(R.astype(np.float64)))).backward()
    for g_, o_, name in zip(grads, os_, ("dx", "dgamma", "dbeta", "dw", "db")):
        assert_close(g_, o_.grad, GRAD_TOL[prec], name)


def test_unknown_output_flags_are_rejected(ctx):
    """Every entry point with output flags rejects unknown bits with TFB_ERR_ARG (-1)
    and records nothing."""
    import ctypes
    from transformer_fwd_bwd_amd import _out
    lib = T.load_library()
    x, w, b = ctx.tensor((4, 8), rnd(191, (4, 8))), ctx.tensor((8, 8), rnd(192, (8, 8))), ctx.tensor((8,), rnd(193, (8,)))
    g1, qkv = ctx.tensor((8,), np.ones(8, np.float32)), ctx.tensor((1, 4, 96), rnd(194, (1, 4, 96)))
    calls = [
        lambda: _out(ctx, lib.tfb_linear_ex, x.h, w.h, b.h, 8),
        lambda: _out(ctx, lib.tfb_matmul_t_ex, x.h, w.h, 8),
        lambda: _out(ctx, lib.tfb_gelu_ex, x.h, 8),
        lambda: _out(ctx, lib.tfb_layernorm_ex, x.h, g1.h, b.h, ctypes.c_float(1e-5), 8),
        lambda: _out(ctx, lib.tfb_causal_attention_ex, qkv.h, 2, 8),
    ]
    for call in calls:
        with pytest.raises(T.TfbError) as e:
            call()
        assert e.value.code == -1
    ctx.tape_reset()
    for t in (x, w, b, g1, qkv):
        t.release()


def test_no_grad_records_nothing(ctx):
    a = ctx.tensor((2, 3), rnd(40, (2, 3)))
    ctx.set_grad_enabled(False)
    y = T.sum_all(T.tanh(a))
    ctx.set_grad_enabled(True)
    ctx.backward(y)            # nothing recorded: only the seed is written
    with pytest.raises(T.TfbError):
        a.grad()
    ctx.tape_reset()
    a.release()


# ----------------------------------------------------------------------------- optimizers
def test_adamw_matches_oracle_over_steps(ctx):
    from oracle import optim as OPT
    shapes = [(37, 65), (65,), (3, 5, 7)]
    params = [rnd(50 + i, s) for i, s in enumerate(shapes)]
    gp = [ctx.tensor(s, p, param=True) for s, p in zip(shapes, params)]
    op = [E.Tensor(p.astype(np.float64)) for p in params]
    gopt = T.AdamW(gp, lr=1e-2, weight_decay=0.1)
    oopt = OPT.AdamW(op, lr=1e-2, weight_decay=0.1)
    for step in range(4):
        grads = [rnd(60 + 10 * step + i, s) for i, s in enumerate(shapes)]
        gopt.zero_grad()
        for t, g in zip(gp, grads):
            Gt = ctx.tensor(g.shape, g)
            ctx.backward(T.sum_all(T.mul(t, Gt)))     # leaves exactly g in t.grad
            ctx.tape_reset()
            Gt.release()
        gopt.step()
        for t, g in zip(op, grads):
            t.grad = g.astype(np.float64)
        oopt.step()
        for t, o in zip(gp, op):
            assert_close(t.numpy(), o.data, 1e-6, f"step {step}")
    gopt.close()
    for t in gp:
        t.release()


def test_sgd(ctx):
    w = ctx.tensor((3,), [1.0, 2.0, 3.0])
    g = ctx.tensor((3,), [0.5, -1.0, 2.0])
    ctx.backward(T.sum_all(T.mul(w, g)))
    T.sgd_step([w], 0.1)
    assert np.allclose(w.numpy(), [0.95, 2.1, 2.8])
    ctx.tape_reset()
    w.release()
    g.release()


@pytest.mark.parametrize("prec", PRECS)
def test_lm_head_with_padded_rows(ctx, prec):
    """A vocabulary-sized LM head (V not a multiple of 64) stores its rows
    padded; the cross-entropy reads them in place and every gradient matches."""
    V, C, rows = 1030, 64, 300
    x, w = rnd(41, (rows, C)), rnd(42, (V, C), 0.2)
    tg = S.random_ids(43, (rows,), V)
    ctx.set_precision(prec)
    xt, wt = ctx.tensor(x.shape, x), ctx.tensor(w.shape, w)
    logits = T.matmul_t(xt, wt)
    loss = T.softmax_cross_entropy(logits, tg)
    ctx.backward(loss)
    ox, ow = E.Tensor(x.astype(np.float64)), E.Tensor(w.astype(np.float64))
    ol = E.matmul_t(ox, ow)
    oloss = E.softmax_cross_entropy(ol, tg)
    oloss.backward()
    tol_f, tol_g = FWD_TOL[prec], GRAD_TOL[prec]
    assert_close(logits.numpy(), ol.data, tol_f, "logits")
    assert abs(loss.item() - oloss.item()) / abs(oloss.item()) <= tol_f
    assert_close(logits.grad(), ol.grad, tol_g, "dlogits")
    assert_close(xt.grad(), ox.grad, tol_g, "dx")
    assert_close(wt.grad(), ow.grad, tol_g, "dw")
    ctx.tape_reset()
    xt.release()
    wt.release()
    ctx.set_precision("fp32")


def test_padded_output_feeds_other_ops(ctx):
    """Another op consuming a padded LM-head output gets a recorded dense copy."""
    check(ctx, "fp32", lambda x, w: T.tanh(T.matmul_t(x, w)), lambda x, w: E.tanh(E.matmul_t(x, w)),
          [rnd(44, (70, 32)), rnd(45, (1100, 32), 0.2)], (70, 1100))


@pytest.mark.parametrize("prec", PRECS)
def test_causal_attention_gpt2_shape(ctx, prec):
    """At the GPT-2 step's own shape (8 x 1024 tokens, 12 heads of 64) -- the fused
    kernels in the bf16 variant, the materialised path in fp32."""
    B, Tn, H, hs = 8, 1024, 12, 64
    qkv = rnd(46, (B, Tn, 3 * H * hs))
    check(ctx, prec, lambda a: T.causal_attention(a, H), lambda a: _attention_oracle(a, H), [qkv],
          (B, Tn, H * hs))
