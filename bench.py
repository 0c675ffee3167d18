"""Training throughput of the GPT-2-124M-shape step on one MI355X.

One step = token + position embedding, 12 pre-LN blocks (LayerNorm, fused
c_attn Linear, causal attention, projection, residual adds, GELU MLP), ln_f,
the weight-tied LM head, SoftmaxCrossEntropy, the full backward replay of the
tape, and one AdamW update of all 124,439,808 parameters -- every step of it in
libtfb's HIP kernels.  Batch 8 x 1024 tokens of uniform random ids (synthetic
data, random N(0, 0.02) weights); inputs are resident in HBM before timing.

Prints one JSON line (see the fields below).  Options:
  --gpus N         only N = 1 is supported (libtfb runs on one GPU)
  --steps K        timed steps (default 20)
  --warmup W       untimed warmup steps (default 5)
  --precision P    bf16 (default: bf16 MFMA operands, fp32 master weights and
                   all other arithmetic in fp32) or fp32
  --no-cpu-baseline  skip timing the CPU oracle
  --copy-probe     first run a plain 1 GiB device-to-device copy (3 times), the
                   known-size reference that HBM byte counters are scaled by
  --decode         time KV-cached generation instead (16 prompts of 768 tokens,
                   256 steps sampled with top-k 40); --steps full generations
                   are timed; --uncached adds generation without the cache

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
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_SUMMARY = {p: os.path.join(ROOT, "profiles", f"gemm_kernel_hbm_traffic_gpt2_124m_train_step_{p}.md")
                   for p in ("bf16", "fp32")}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--precision", choices=["bf16", "fp32"], default="bf16")
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--seq", type=int, default=1024)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seq", type=int, default=1024)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time KV-cached generation (16 prompts of 768 tokens, 256 sampled steps) instead")
    ap.add_argument("--uncached", action="store_true", help="with --decode: also time generation without the cache")
    return ap.parse_args()


def cpu_baseline(seq: int):
    """The float64 oracle, untuned, on this host's cores: one fwd + bwd + AdamW step of
    the same GPT-2-124M shape on ONE sequence of `seq` tokens (a bounded sample)."""
    import numpy as np

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
    return {"value": seq / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"one fwd+bwd+AdamW step of the float64 oracle on 1 x {seq} tokens, GPT-2-124M shape "
                      f"({dt:.1f} s; numpy/OpenBLAS on {cores} threads)"}


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


def decode_bench(args):
    """KV-cached generation at the GPT-2-124M shape: 16 prompts of 768 tokens, then 256
    steps sampled with top-k 40 at temperature 1 (uniforms drawn beforehand).  --warmup
    short generations, then --steps timed full generations; the prefill alone is timed
    the same way so that the per-step cost of decoding can be separated from it."""
    import torch

    import synthetic as S
    import transformer_fwd_bwd_amd as T
    from transformer_fwd_bwd_amd import gpt as G

    s, params, prompts, u = S.gpt2_infer()
    B, Pn = prompts.shape
    n_new = u.shape[1]
    ctx = T.Context(arena_bytes=int(os.environ.get("TFB_ARENA_GB", "64")) << 30, precision=args.precision)
    model = G.Gpt(ctx, s.n_layer, s.n_head, params)
    del params
    pd, ud = torch.from_numpy(prompts).to("cuda:0"), torch.from_numpy(u).to("cuda:0")
    for _ in range(args.warmup):
        model.generate(pd[:, :64].contiguous(), 4, ud[:, :4].contiguous(), 40, 1.0)
    torch.cuda.synchronize()

    def timed(fn):
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps

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
    out = {
        "metric": "KV-cached generation: sampled tokens/s (16 x 768-token prompts, 256 steps, top-k 40)",
        "value": round(B * n_new / t_gen, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_generation": round(t_gen * 1e3, 2),
        "prefill_ms": round(t_pre * 1e3, 2),
        "decode_ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "dtype": args.precision,
        "data": "synthetic",
        "config": {"workload": "gpt2-124m-shape KV-cached generation", "batch": B, "prompt": Pn, "new_tokens": n_new},
    }
    if args.uncached:
        t_unc = timed(lambda: model.generate_uncached(pd, n_new, ud, 40, 1.0))
        out["uncached_ms_per_generation"] = round(t_unc * 1e3, 2)
        out["cached_speedup"] = round(t_unc / t_gen, 2)
    ctx.close()
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: libtfb runs on exactly one GPU (asked for --gpus {args.gpus}); "
              "data parallelism across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)
    if args.decode:
        decode_bench(args)
        return
    import numpy as np
    import torch

    import synthetic as S
    import transformer_fwd_bwd_amd as T
    from transformer_fwd_bwd_amd import gpt as G

    if args.copy_probe:
        copy_probe()
    B, L = args.batch, args.seq
    s, params, ids = S.gpt2(batch=B, seq=L)
    ctx = T.Context(arena_bytes=int(os.environ.get("TFB_ARENA_GB", "64")) << 30, precision=args.precision)
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
    for i in range(args.warmup):
        loss = step()
        if i == 0:
            first_loss = loss.item()
        ctx.tape_reset()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
        ctx.tape_reset()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / args.steps * 1e3
    tokens_per_s = B * L * args.steps / dt

    # the contraction kernels, timed with HIP events on the library's stream over K more steps
    ctx.profile_begin()
    for _ in range(args.steps):
        loss = step()
        last_loss = loss.item() if _ == args.steps - 1 else None
        ctx.tape_reset()
    gemm_ms, gemm_flops, launches = ctx.profile_end()
    achieved = gemm_flops / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[args.precision]

    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.precision,
        "data": "synthetic",
        "config": {"workload": "gpt2-124m-shape train step (fwd+bwd+AdamW)", "global_batch": B, "seq_len": L,
                   "parallelism": "none (1 GPU)",
                   "variant": "bf16 MFMA operands, fp32 master/accumulate" if args.precision == "bf16"
                   else "fp32 throughout"},
        "roofline": {"bound": "mfma", "kernel": "gemm_kernel (all contraction launches)",
                     "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": gemm_traffic(args.precision) if (B, L) == (8, 1024) else None,
                     "gemm_ms_per_step": round(gemm_ms / args.steps, 3),
                     "gemm_tflop_per_step": round(gemm_flops / args.steps / 1e12, 4),
                     "launches_per_step": launches // args.steps},
        "loss_first_step": round(first_loss, 5) if first_loss is not None else None,
        "loss_last_step": round(last_loss, 5) if last_loss is not None else None,
    }
    ctx.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample_seq)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
