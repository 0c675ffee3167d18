"""Training throughput of the GPT-2-124M-shape step on one MI355X.

One step = token + position embedding, 12 pre-LN blocks (LayerNorm, fused
c_attn Linear, causal attention, projection, residual adds, GELU MLP), ln_f,
the weight-tied LM head, SoftmaxCrossEntropy, the full backward replay of the
tape, and one AdamW update of all 124,439,808 parameters -- every step of it in
libtfb's HIP kernels.  Batch 8 x 1024 tokens of uniform random ids (synthetic
data, random N(0, 0.02) weights); inputs are resident in HBM before timing.

Prints one JSON line.  `value` is the bf16-MFMA / fp32-master variant's
training tokens/s (--precision fp32 makes the fp32 variant the headline).
Beside it the line carries:
  roofline      the contraction family (the dominant kernel, MFMA-bound) with
                `families`: every timed kernel family's achieved rate against
                its own bound (MFMA peak for the contractions and the fused
                attention, HBM peak for the rest), all from HIP events on the
                library's stream over --steps extra steps; `hbm_reference`: what
                a plain copy and a plain fill reach on this GPU
  fp32          the fp32 variant of the same step: ms/step, tokens/s and its
                contraction roofline against the fp32 MFMA peak
  decode        KV-cached generation at the same shape (16 prompts of 768
                tokens, 256 steps, top-k 40): sampled tokens/s, ms per decode
                step and its algorithmic bytes per step against HBM
  cpu_baseline  the float64 oracle on this host's cores (a bounded sample)
Options:
  --gpus N         only N = 1 is supported (libtfb runs on one GPU)
  --steps K        timed training steps (default 20); the fp32 leg times
                   min(K, 8) steps and the decode leg one generation per 10 K
  --warmup W       untimed warmup steps (default 5; fp32 leg min(W, 2))
  --precision P    headline variant: bf16 (default) or fp32
  --no-fp32 / --no-decode / --no-cpu-baseline   skip a leg
  --copy-probe     first run a plain 1 GiB device-to-device copy (3 times), the
                   known-size reference that HBM byte counters are scaled by
  --decode         print the decode leg alone as the line (--steps full
                   generations); --uncached adds generation without the cache

roofline.traffic is the contraction kernel's HBM bytes per launch as read by the
FETCH_SIZE and WRITE_SIZE counters (scaled by the copy probe), taken from the
committed counter summary when that summary was made from the same gemm.hip;
otherwise null.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "train tokens/sec (fwd+bwd+AdamW) at GPT-2-124M shape; MFMA util %, HBM GB/s"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0                            # MI355X HBM3E, published
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARY = {p: os.path.join(ROOT, "profiles", f"gemm_hbm_traffic_gpt2_124m_train_step_{p}.md")
                   for p in ("bf16", "fp32")}
FAMILY_NAMES = {
    "gemm": "gemm_kernel + gemm_dma_kernel (MatMul family, split-K reductions included)", "attn_fwd": "attn_fwd_k (fused causal attention)",
    "attn_bwd": "attn_dq_k + attn_dkv_k (fused attention backward)", "ce": "ce_fwd_grad4_k / ce kernels",
    "adamw": "adamw_k", "ln_fwd": "ln_fwd4_k", "ln_bwd": "ln_bwd_fused4_k", "gelu_fwd": "gelu forward",
    "gelu_bwd": "gelu backward", "gemv": "gemv_k + gemv_reduce_ln_k + gemv_nt_k (decode Linears and LM head)",
    "kv_attend": "kv_attend_part_k (cached attention)", "sample": "sample_topk_reg_k",
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--precision", choices=["bf16", "fp32"], default="bf16")
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--seq", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp32", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-sample-seq", type=int, default=1024)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="print the KV-cached generation leg alone (16 prompts of 768 tokens, 256 sampled steps)")
    ap.add_argument("--uncached", action="store_true", help="with --decode: also time generation without the cache")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(seq: int):
    """The float64 oracle, untuned, on this host's cores: one fwd + bwd + AdamW step of
    the same GPT-2-124M shape on ONE sequence of `seq` tokens (a bounded sample)."""
    import synthetic as S
    from oracle import models as M
    from oracle import optim as OPT

    s, params, ids = S.gpt2(batch=1, seq=seq)
    t0 = time.perf_counter()
    P = M.as_tensors(params)
    loss, _ = M.gpt_loss(P, ids, s.n_layer, s.n_head)
    loss.backward()
    OPT.AdamW(list(P.values()), lr=1e-3, weight_decay=0.01).step()
    dt = time.perf_counter() - t0
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    model = cpu_model()
    return {"value": seq / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": model,
            "sample": f"one fwd+bwd+AdamW step of the float64 oracle on 1 x {seq} tokens, GPT-2-124M shape "
                      f"({dt:.1f} s; numpy/OpenBLAS on {cores} threads of {model})"}


def gemm_traffic(precision: str):
    """HBM bytes per contraction launch from the committed counter summary, if it was
    taken on the current gemm.hip (its sha256 is recorded there); else None."""
    import hashlib
    path = TRAFFIC_SUMMARY[precision]
    if not os.path.exists(path):
        return None
    src = os.path.join(ROOT, "transformer_fwd_bwd_amd", "csrc", "gemm.hip")
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    fields = {}
    for line in open(path):
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("gemm.hip sha256") != digest:
        return None
    try:
        return int(fields["bytes per launch"])
    except (KeyError, ValueError):
        return None


def copy_probe():
    import torch
    n = 1 << 28                                   # 2^28 floats = 1 GiB each way
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)                   # one streaming kernel: reads 1 GiB, writes 1 GiB
    torch.cuda.synchronize()
    del src, dst


def hbm_reference():
    """Achieved rate of plain streaming kernels on this GPU (torch's own, 1 GiB per
    stream): the practical ceiling the bandwidth-bound families are measured against
    beside the 8 TB/s published peak."""
    import torch
    n = 1 << 28
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    out = {}
    for name, fn, nbytes in (("copy_1r1w", lambda: b.copy_(a), 8 * n), ("fill_1w", lambda: b.fill_(1.0), 4 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_gbs"] = round(nbytes / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def families(ctx, steps: int, precision: str):
    """Per kernel family: achieved rate against its bound, from the profile just ended."""
    import transformer_fwd_bwd_amd as T
    out = {}
    for name, (ms, work, n) in ctx.profile_families().items():
        if ms <= 0:
            continue
        if T.PROF_UNIT.get(name) == "flop":
            ach, peak, unit, bound = work / (ms * 1e-3) / 1e12, PEAK_TFLOPS[precision], "TFLOP/s", "mfma"
            per = {"tflop_per_step": round(work / steps / 1e12, 4)}
        else:
            ach, peak, unit, bound = work / (ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
            per = {"gb_per_step": round(work / steps / 1e9, 4)}
        out[name] = {"kernel": FAMILY_NAMES.get(name, name), "bound": bound, "achieved": round(ach, 2),
                     "peak": peak, "unit": unit, "frac": round(ach / peak, 4),
                     "ms_per_step": round(ms / steps, 4), "launches_per_step": round(n / steps, 2), **per}
    return out


def train_leg(precision: str, B: int, L: int, steps: int, warmup: int, arena_gb: int):
    """W warmup steps, K timed steps, then K more steps with every kernel family
    bracketed by HIP events (the roofline figures)."""
    import torch

    import synthetic as S
    import transformer_fwd_bwd_amd as T
    from transformer_fwd_bwd_amd import gpt as G

    s, params, ids = S.gpt2(batch=B, seq=L)
    ctx = T.Context(arena_bytes=arena_gb << 30, precision=precision)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    del params
    opt = T.AdamW(model.param_list, lr=1e-4, weight_decay=0.01)
    ids_dev = torch.from_numpy(ids).to("cuda:0")
    inputs, targets = G.split_ids(ids_dev)
    ctx.sync()

    def step():
        loss, _ = model.loss(inputs, targets)
        opt.zero_grad()
        ctx.backward(loss)
        opt.step()
        return loss

    first_loss = None
    for i in range(warmup):
        loss = step()
        if i == 0:
            first_loss = loss.item()
        ctx.tape_reset()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(steps):
        step()
        ctx.tape_reset()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0

    ctx.profile_begin()
    last_loss = None
    for i in range(steps):
        loss = step()
        if i == steps - 1:
            last_loss = loss.item()
        ctx.tape_reset()
    gemm_ms, gemm_flops, launches = ctx.profile_end()
    fam = families(ctx, steps, precision)
    opt.close()
    ctx.close()
    del model, opt, ctx
    torch.cuda.empty_cache()
    return {"dt": dt, "ms": dt / steps * 1e3, "tokens_per_s": B * L * steps / dt, "gemm_ms": gemm_ms,
            "gemm_flops": gemm_flops, "launches": launches, "families": fam,
            "first_loss": first_loss, "last_loss": last_loss}


def gemm_roofline(r, precision: str, steps: int, traffic):
    achieved = r["gemm_flops"] / (r["gemm_ms"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[precision]
    return {"bound": "mfma", "kernel": "gemm_kernel + gemm_dma_kernel (all contraction launches, split-K reductions included)",
            "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "gemm_ms_per_step": round(r["gemm_ms"] / steps, 3),
            "gemm_tflop_per_step": round(r["gemm_flops"] / steps / 1e12, 4),
            "launches_per_step": r["launches"] // steps}


def decode_bytes_per_step(s, B: int, prompt: int, n_new: int, precision: str) -> float:
    """Algorithmic HBM bytes of one decode step, averaged over the generation: every
    block weight and the tied LM-head table once (in the form the products read: bf16
    copies in the bf16 variant), the cached keys and values of all earlier positions
    (fp32, or bf16 in the bf16 variant), and the logits written and read by the sampler."""
    C, V, nl = s.n_embd, s.vocab, s.n_layer
    w_block = nl * (C * 3 * C + C * C + C * 4 * C + 4 * C * C)
    ew = 2 if precision == "bf16" else 4
    weights = ew * (w_block + V * C)
    mean_len = prompt + (n_new - 1) / 2.0          # positions 0..pos read at pos = prompt-1+i, i < n_new
    kv = nl * B * mean_len * C * 2 * ew             # the cache holds the variant's operand type
    logits = B * V * 4 * 2
    return weights + kv + logits


def decode_leg(precision: str, gens: int, warmup: int, arena_gb: int, uncached: bool = False):
    """KV-cached generation at the GPT-2-124M shape: 16 prompts of 768 tokens, then 256
    steps sampled with top-k 40 at temperature 1 (uniforms drawn beforehand).  `warmup`
    short generations, then `gens` timed full generations; the prefill alone is timed
    the same way so that the per-step cost of decoding can be separated from it; then
    one more generation with the kernel families of its decode steps bracketed."""
    import torch

    import synthetic as S
    import transformer_fwd_bwd_amd as T
    from transformer_fwd_bwd_amd import gpt as G

    s, params, prompts, u = S.gpt2_infer()
    B, Pn = prompts.shape
    n_new = u.shape[1]
    ctx = T.Context(arena_bytes=arena_gb << 30, precision=precision)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    del params
    pd, ud = torch.from_numpy(prompts).to("cuda:0"), torch.from_numpy(u).to("cuda:0")
    for _ in range(max(warmup, 1)):
        model.generate(pd[:, :64].contiguous(), 4, ud[:, :4].contiguous(), 40, 1.0)
    torch.cuda.synchronize()

    def timed(fn):
        t0 = time.perf_counter()
        for _ in range(gens):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / gens

    def prefill():
        kv = T.KvCache(ctx, s.n_layer, B, Pn + n_new - 1, s.n_embd)
        ctx.set_grad_enabled(False)
        model.prefill(pd[:, :-1].contiguous(), kv)
        ctx.tape_reset()
        ctx.set_grad_enabled(True)
        kv.close()

    t_gen = timed(lambda: model.generate(pd, n_new, ud, 40, 1.0))
    t_pre = timed(prefill)
    step_ms = (t_gen - t_pre) / n_new * 1e3
    bps = decode_bytes_per_step(s, B, Pn, n_new, precision)
    ach = bps / (step_ms * 1e-3) / 1e9
    # the families over decode steps 1..n_new-1 only (profiling starts once step 0 is queued)
    model.generate(pd, n_new, ud, 40, 1.0, on_step=lambda i, lg, tk: ctx.profile_begin() if i == 0 else None)
    ctx.profile_end()
    fam = families(ctx, n_new - 1, precision)
    out = {
        "metric": "KV-cached generation: sampled tokens/s (16 x 768-token prompts, 256 steps, top-k 40)",
        "value": round(B * n_new / t_gen, 1), "unit": "tokens/s", "dtype": precision,
        "ms_per_generation": round(t_gen * 1e3, 2), "prefill_ms": round(t_pre * 1e3, 2),
        "decode_ms_per_step": round(step_ms, 4),
        "decode_tokens_per_s": round(B / (step_ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "one decode step (all its kernels)", "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "gb_per_step": round(bps / 1e9, 4), "families": fam},
        "config": {"workload": "gpt2-124m-shape KV-cached generation", "batch": B, "prompt": Pn, "new_tokens": n_new},
    }
    if uncached:
        t_unc = timed(lambda: model.generate_uncached(pd, n_new, ud, 40, 1.0))
        out["uncached_ms_per_generation"] = round(t_unc * 1e3, 2)
        out["cached_speedup"] = round(t_unc / t_gen, 2)
    ctx.close()
    del model, ctx
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: libtfb runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "data parallelism across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    arena_gb = int(os.environ.get("TFB_ARENA_GB", "64"))
    if args.decode:
        d = decode_leg(args.precision, args.steps, args.warmup, 32, args.uncached)
        d.update({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                  "data": "synthetic"})
        print(json.dumps(d), flush=True)
        return
    if args.copy_probe:
        copy_probe()
    B, L = args.batch, args.seq
    r = train_leg(args.precision, B, L, args.steps, args.warmup, arena_gb)
    out = {
        "metric": METRIC,
        "value": round(r["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.precision,
        "data": "synthetic",
        "config": {"workload": "gpt2-124m-shape train step (fwd+bwd+AdamW)", "global_batch": B, "seq_len": L,
                   "parallelism": "none (1 GPU)",
                   "variant": "bf16 MFMA operands, fp32 master/accumulate" if args.precision == "bf16"
                   else "fp32 throughout"},
        "roofline": gemm_roofline(r, args.precision, args.steps,
                                  gemm_traffic(args.precision) if (B, L) == (8, 1024) else None),
        "loss_first_step": round(r["first_loss"], 5) if r["first_loss"] is not None else None,
        "loss_last_step": round(r["last_loss"], 5) if r["last_loss"] is not None else None,
    }
    out["roofline"]["families"] = r["families"]
    out["roofline"]["hbm_reference"] = hbm_reference()
    if args.precision == "bf16" and not args.no_fp32:
        k32, w32 = min(args.steps, 8), min(args.warmup, 2)
        r32 = train_leg("fp32", B, L, k32, w32, arena_gb)
        out["fp32"] = {"variant": "fp32 throughout (the pages' arithmetic)", "steps": k32, "warmup": w32,
                       "ms_per_step": round(r32["ms"], 3), "tokens_per_s": round(r32["tokens_per_s"], 1),
                       "roofline": gemm_roofline(r32, "fp32", k32, None),
                       "families": r32["families"]}
    if not args.no_decode:
        gens = max(1, args.steps // 10)
        d = decode_leg(args.precision, gens, 1, 32)
        out["decode"] = {k: d[k] for k in ("value", "unit", "ms_per_generation", "prefill_ms", "decode_ms_per_step",
                                           "decode_tokens_per_s", "roofline", "config")}
        out["decode"]["generations_timed"] = gens
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_seq)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
