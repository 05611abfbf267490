"""Benchmark of the fused attention-KL hot path on one MI355X.

One step = forward (KL, LSE1, LSE2) + backward (dQ1, dK1, dQ2, dK2) of the
causal 64K-context workload: B=1, H=32, N_Q=N_K=65536, D=128, bf16 inputs,
fp32 accumulation, synthetic Gaussian teacher/student tensors already resident
in HBM.  Throughput is algorithmic TFLOP/s over exact visible (query, key)
pairs: 4*D flop per pair forward, 12*D backward.

Also reported: per-kernel HIP-event timings, the roofline of the dominant
kernel, the split-K forward on the 512K-key workload, and the fp64 CPU oracle
timed on a bounded sample of the same workload on this host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn-KL fwd and fwd+bwd TFLOP/s + ms at 64K ctx, 32 heads, d=128 bf16"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak (published)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="causal_64k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-splitk", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    return ap.parse_args()


def cpu_baseline(w, q1, k1, q2, k2, target_s: float):
    """Time the fp64 oracle (fwd + bwd) on evenly spaced rows of head (0, 0)."""
    import numpy as np
    import oracle
    if not os.path.exists(oracle.LIB_PATH):
        oracle.build(force=False)
    f = lambda t: t[0, 0].to("cpu").double().numpy()
    hq1, hk1, hq2, hk2 = f(q1), f(k1), f(q2), f(k2)
    g = 1.0 / (w.B * w.H * w.NQ)

    def run(nrows):
        rows = np.linspace(0, w.NQ - 1, nrows).round().astype(np.int64)
        off = w.NK - w.NQ
        pairs = int(np.sum(np.minimum(w.NK, rows + off + 1))) if w.causal else nrows * w.NK
        t0 = time.perf_counter()
        oracle.bwd(hq1, hk1, hq2, hk2, w.scale, w.causal, np.full(nrows, g), rows=rows)
        return time.perf_counter() - t0, pairs

    dt, pairs = run(16)
    per_pair = dt / pairs
    nrows = int(max(16, min(w.NQ, 16 * target_s / max(dt, 1e-6))))
    dt, pairs = run(nrows)
    flops = pairs * 16 * w.D
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle fwd+bwd on {nrows} evenly spaced query rows of head (0,0) of {w.name} "
                  f"({pairs} visible pairs, {dt:.1f} s; flops counted as 16*D per pair)",
        "seconds": dt,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(each GPU's share would run the same kernels independently).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import attention_kl_divergence_online_amd as skl

    w = synth.get(args.workload)
    dev = "cuda"
    torch.cuda.init()
    q1, k1, q2, k2 = synth.make_inputs(w, device=dev)
    g = synth.upstream_grad(w, dev)
    kl, l1, l2 = (torch.empty((w.B, w.H, w.NQ), dtype=torch.float32, device=dev) for _ in range(3))
    grads = (torch.empty_like(q1, dtype=torch.float32), torch.empty_like(k1, dtype=torch.float32),
             torch.empty_like(q2, dtype=torch.float32), torch.empty_like(k2, dtype=torch.float32))
    ws = torch.empty(max(16, skl.bwd_workspace_size(q1, k1, w.scale, w.causal)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        skl.streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal, out=(kl, l1, l2))
        if ev is not None:
            ev[1].record()
        skl.streamkl_bwd_prepare(q1, k1, g, w.scale, w.causal, workspace=ws)
        if ev is not None:
            ev[2].record()
        skl.streamkl_bwd_dk(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal, workspace=ws,
                            out=(grads[1], grads[3]))
        if ev is not None:
            ev[3].record()
        skl.streamkl_bwd_dq(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal, workspace=ws,
                            out=(grads[0], grads[2]))
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for k in range(args.steps):
        step(evs[k])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    per = {"fwd": 0.0, "bwd_prepare": 0.0, "bwd_dk": 0.0, "bwd_dq": 0.0}
    for e in evs:
        per["fwd"] += e[0].elapsed_time(e[1])
        per["bwd_prepare"] += e[1].elapsed_time(e[2])
        per["bwd_dk"] += e[2].elapsed_time(e[3])
        per["bwd_dq"] += e[3].elapsed_time(e[4])
    per = {k: v / args.steps for k, v in per.items()}
    fwd_ms = per["fwd"]
    bwd_ms = per["bwd_prepare"] + per["bwd_dk"] + per["bwd_dq"]

    pairs = w.visible_pairs()
    fwd_flop = 4 * w.D * pairs
    bwd_flop = 12 * w.D * pairs
    tflops = (fwd_flop + bwd_flop) / (ms_step * 1e-3) / 1e12

    # Roofline of the longest kernel.  Algorithmic flop per launch: forward 4*D
    # per visible pair; each backward pass 8*D per pair (its recompute of both
    # logit tiles, 4*D, plus its two gradient products, 4*D).
    kern_flop = {"fwd": fwd_flop, "bwd_dk": 8 * w.D * pairs, "bwd_dq": 8 * w.D * pairs}
    dom = max(kern_flop, key=lambda k: per[k])
    achieved = kern_flop[dom] / (per[dom] * 1e-3) / 1e12
    kernel_names = {"fwd": "fwd_kernel<bf16,128,false>", "bwd_dk": "bwd_kernel<bf16,128,true>",
                    "bwd_dq": "bwd_kernel<bf16,128,false>"}

    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "NQ": w.NQ, "NK": w.NK, "D": w.D,
                   "causal": w.causal, "inputs": "bf16", "accumulate": "fp32"},
        "fwd_ms": round(fwd_ms, 3),
        "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_ms": round(bwd_ms, 3),
        "bwd_tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
        "kernel_ms": {k: round(v, 3) for k, v in per.items()},
        "wall_s_timed": round(wall, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": kernel_names[dom],
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
    }

    if not args.no_splitk:
        out["splitk"] = splitk_bench(skl, synth, torch, args)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q1, k1, q2, k2, args.cpu_seconds)

    print(json.dumps(out), flush=True)


def splitk_bench(skl, synth, torch, args):
    """Split-K forward on the 512K-key, 1024-query workload (64 chunks)."""
    w = synth.get("splitk_512k")
    q1, k1, q2, k2 = synth.make_inputs(w, device="cuda")
    out = tuple(torch.empty((w.B, w.H, w.NQ), dtype=torch.float32, device="cuda") for _ in range(3))
    ws = torch.empty(skl.fwd_splitk_workspace_size(q1, k1, w.splits, w.scale, w.causal), dtype=torch.uint8,
                     device="cuda")
    for _ in range(args.warmup):
        skl.streamkl_fwd_splitk(q1, k1, q2, k2, w.splits, w.scale, w.causal, workspace=ws, out=out)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        skl.streamkl_fwd_splitk(q1, k1, q2, k2, w.splits, w.scale, w.causal, workspace=ws, out=out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    flop = 4 * w.D * w.visible_pairs()
    res = {"workload": w.name, "splits": w.splits, "ms": round(ms, 3),
           "tflops": round(flop / (ms * 1e-3) / 1e12, 2)}
    del q1, k1, q2, k2, ws
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
