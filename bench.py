"""Benchmark of the fused attention-KL hot path on one MI355X.

One step = forward (KL, LSE1, LSE2) + backward (dQ1, dK1, dQ2, dK2) of the
causal 64K-context workload: B=1, H=32, N_Q=N_K=65536, D=128, bf16 inputs,
fp32 accumulation, synthetic Gaussian teacher/student tensors already resident
in HBM.  Throughput is algorithmic TFLOP/s over exact visible (query, key)
pairs: 4*D flop per pair forward, 12*D backward.

Also reported: per-kernel HIP-event timings, the roofline of the dominant
kernel (algorithmic flop per launch over its average duration), the other
four workloads of the metric ("configs": tiny fp32, causal 4K, non-causal
16K, the split-K forward over 512K keys and the backward over 128K keys),
the same step with the inputs rounded to fp8 e4m3 ("fp8"), and the fp64 CPU
oracle timed on a bounded sample of the same workload on this host's cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn-KL fwd and fwd+bwd TFLOP/s + ms at 64K ctx, 32 heads, d=128 bf16"
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "attention_kl_causal_64k_hbm_traffic.json")
COPY_BYTES = 1 << 30
KERNELS = {  # bench key -> kernel names as rocprofv3 reports them (mangled or demangled)
    "fwd": ("_ZN3skl11fwd2_kernelILi128ELb0ELi8ELi128ELb0EEEvNS_9FwdParamsE",
            "void skl::fwd2_kernel<128, false, 8, 128, false>"),
    "bwd_dk": ("_ZN3skl11bwd4_kernelILi128ELb1ELi0ELb0EEEvNS_9BwdParamsE",
               "void skl::bwd4_kernel<128, true, 0, false>"),
    "bwd_dq": ("_ZN3skl11bwd4_kernelILi128ELb0ELi0ELb0EEEvNS_9BwdParamsE",
               "void skl::bwd4_kernel<128, false, 0, false>"),
    "fwd_split": ("_ZN3skl11fwd2_kernelILi128ELb1ELi8ELi128ELb0EEEvNS_9FwdParamsE",
                  "void skl::fwd2_kernel<128, true, 8, 128, false>"),
}


def kernel_source_hash() -> str:
    """sha256 over the kernel sources; counter records are valid only for this hash."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_kl_divergence_online_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def summarize_traffic(fetch_csv: str, write_csv: str) -> None:
    """Per-launch HBM bytes of the bench kernels from two rocprofv3 --pmc runs.

    FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for the calibration copy of COPY_BYTES (the device copy
    kernel whose FETCH_SIZE is closest to COPY_BYTES)."""
    import csv

    def load(path, counter):
        per = {}
        copy_vals = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            name = r["Kernel_Name"]
            for key, syms in KERNELS.items():
                if name.startswith(syms):
                    per.setdefault(key, []).append(v)
            if "copy" in name.lower() or "elementwise" in name.lower():
                copy_vals.append(v)
        ref = min(copy_vals, key=lambda v: abs(v - COPY_BYTES)) if copy_vals else None
        return per, ref

    fetch, fref = load(fetch_csv, "FETCH_SIZE")
    write, wref = load(write_csv, "WRITE_SIZE")
    if not fref or not wref:
        raise SystemExit("calibration copy not found in the counter CSVs (run bench.py --calibrate-copy)")
    fs, wsc = COPY_BYTES / fref, COPY_BYTES / wref
    rec = {"source_sha256": kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "fetch_scale": fs, "write_scale": wsc, "kernels": {}}
    for key in KERNELS:
        if key in fetch and key in write:
            f = sum(fetch[key]) / len(fetch[key]) * fs
            w = sum(write[key]) / len(write[key]) * wsc
            rec["kernels"][key] = {"fetch_bytes": f, "write_bytes": w, "bytes": f + w}
    os.makedirs(os.path.dirname(TRAFFIC_RECORD), exist_ok=True)
    with open(TRAFFIC_RECORD, "w") as fo:
        json.dump(rec, fo, indent=1)
    print(json.dumps(rec, indent=1))


def recorded_traffic(key: str):
    """HBM bytes per launch of kernel `key` from the committed record, or None if
    absent or taken on different kernel sources."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    k = rec.get("kernels", {}).get(key)
    return None if k is None else k["bytes"]


def summarize_counters(csvs, out_path: str) -> None:
    """Utilisation table of the bench kernels from rocprofv3 --pmc counter CSVs.

    MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs * kernel cycles), with kernel
    cycles = GRBM_GUI_ACTIVE / XCDs; the per-wave shares divide SQ_* cycle counts
    (in units of 4 cycles) by SQ_WAVE_CYCLES."""
    import csv
    vals = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            for key, syms in KERNELS.items():
                if r["Kernel_Name"].startswith(syms):
                    vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    simds, xcds = 1024, 8
    lines = [f"{'kernel':9s} {'ms@2.4G':>7s} {'MFMA busy':>10s} {'VALU/wave':>10s} {'wait/wave':>10s} "
             f"{'LDS conflict':>13s} {'VALU lane-op/pair':>18s} {'exp/pair':>9s}"]
    import synth
    workload_of = {"fwd_split": "splitk_512k"}  # per-pair figures use the kernel's own workload
    for key in KERNELS:
        pairs = synth.get(workload_of.get(key, "causal_64k")).visible_pairs()
        d = {k: sum(v) / len(v) for k, v in vals.get(key, {}).items()}
        if "GRBM_GUI_ACTIVE" not in d:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / xcds
        wc = d.get("SQ_WAVE_CYCLES", float("nan"))
        g = lambda name: d.get(name, float("nan"))
        lines.append(
            f"{key:9s} {cyc / 2.4e6:7.1f} {g('SQ_VALU_MFMA_BUSY_CYCLES') / (simds * cyc):10.1%} "
            f"{g('SQ_ACTIVE_INST_VALU') / wc:10.1%} {g('SQ_WAIT_INST_ANY') / wc:10.1%} "
            f"{g('SQ_LDS_BANK_CONFLICT') / g('SQ_LDS_IDX_ACTIVE'):13.1%} "
            f"{(g('SQ_INSTS_VALU') - g('SQ_INSTS_MFMA')) * 64 / pairs:18.2f} "
            f"{g('SQ_INSTS_VALU_TRANS_F32') * 64 / pairs:9.2f}")
    text = "\n".join(lines) + "\n"
    with open(out_path, "w") as fo:
        fo.write(text)
    print(text)
    # Co-execution of the matrix and vector units, when the counters are present:
    # per SIMD, as shares of the kernel's cycles.  MFMA busy and co-exec divide
    # SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES by SIMDs x kernel
    # cycles; VALU active is 2 waves per SIMD x SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES;
    # idle = 1 - (MFMA busy + VALU active - co-exec).
    rows = []
    for key in KERNELS:
        d = {k: sum(v) / len(v) for k, v in vals.get(key, {}).items()}
        if "SQ_VALU_MFMA_COEXEC_CYCLES" not in d or "GRBM_GUI_ACTIVE" not in d:
            continue
        cyc = d["GRBM_GUI_ACTIVE"] / xcds
        mf = d["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc)
        co = d["SQ_VALU_MFMA_COEXEC_CYCLES"] / (simds * cyc)
        va = 2 * d.get("SQ_ACTIVE_INST_VALU", float("nan")) / d["SQ_WAVE_CYCLES"]
        lw = d.get("SQ_WAIT_INST_LDS", float("nan")) / d["SQ_WAVE_CYCLES"]
        rows.append(f"{key:9s} {mf:10.1%} {co:8.1%} {co / mf:13.1%} {va:11.1%} {mf - co:10.1%} {va - co:10.1%} "
                    f"{1 - (mf + va - co):6.1%} {lw:14.1%}")
    if rows:
        head = (f"{'kernel':9s} {'MFMA busy':>10s} {'co-exec':>8s} {'co-exec/MFMA':>13s} {'VALU active':>11s} "
                f"{'MFMA only':>10s} {'VALU only':>10s} {'idle':>6s} {'LDS wait/wave':>14s}")
        text = "\n".join([head] + rows) + "\n"
        with open(out_path.replace("_counters.table", "_coexec.table"), "w") as fo:
            fo.write(text)
        print(text)


PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix peak (published)
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 matrix peak (published)
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix peak (published)
# The five workloads the metric is quoted on, by role: C1 tiny fp32 (parity
# size), C2 short causal, C3 long non-causal with large KL, C4 the 64K causal
# headline (the main line above), C5 the split-K forward over 512K keys and
# the short-query backward over 128K keys.
CONFIGS = (("C1", "tiny_fp32"), ("C2", "causal_4k"), ("C3", "noncausal_16k"), ("C5_bwd", "splitk_bwd_128k"))
PEAK_HBM_GBS = 8000.0


def progress(msg: str) -> None:
    """One line per finished section on stderr (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="causal_64k")
    ap.add_argument("--fp8", action="store_true",
                    help="round the workload's inputs to e4m3 and time the fp8 path (the line then reports "
                         "inputs fp8_e4m3; fractions stay against the bf16/fp16 matrix peak)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-splitk", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the other four workloads of the metric (C1 tiny_fp32, C2 causal_4k, "
                         "C3 noncausal_16k, C5 splitk_512k forward and splitk_bwd_128k)")
    ap.add_argument("--no-small-workspace", action="store_true",
                    help="accepted for older command lines; the backward's workspace is O(B*H) and "
                         "needs no smaller-workspace timing")
    ap.add_argument("--other-configs", action="store_true",
                    help="also time forward and backward on the workloads outside the metric "
                         "(shortq_bwd_64k, causal_16k_d64, causal_4k_fp32), the decode split-K "
                         "forward and the packed variable-length batches (varlen_mix, varlen_short), and "
                         "report them under \"other_configs\"")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    ap.add_argument("--materialised-heads", type=int, default=2,
                    help="(b, h) slices on which to time the PyTorch materialise-then-reduce baseline "
                         "(scaled to the whole batch; 0 skips it)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device copy first (scale reference for HBM byte counters)")
    ap.add_argument("--summarize-counters", nargs="+", metavar="CSV",
                    help="print the utilisation table of rocprofv3 --pmc counter CSVs to "
                         "profiles/attention_kl_causal_64k_counters.table (and, given the co-execution "
                         "counters, profiles/attention_kl_causal_64k_coexec.table) and exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a "
                         "--calibrate-copy run into the traffic record under profiles/ and exit")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unreadable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


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
    nrows = int(max(16, min(w.NQ, 16 * target_s / max(dt, 1e-6))))
    dt, pairs = run(nrows)
    flops = pairs * 16 * w.D
    total = w.visible_pairs()
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.threads(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"fp64 oracle fwd+bwd on {nrows} evenly spaced query rows of head (0,0) of {w.name} "
                  f"({pairs} visible pairs, {dt:.1f} s; flops counted as 16*D per pair)",
        "seconds": dt,
        # The whole problem at the sample's rate (rows of a head cost in
        # proportion to their visible pairs), labelled as the extrapolation it is.
        "full_problem_seconds_extrapolated": round(dt * total / pairs, 1),
        "extrapolation": f"sample rate x {total} visible pairs of all {w.B * w.H} heads",
    }


def main():
    args = parse()
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters,
                           os.path.join(ROOT, "profiles", "attention_kl_causal_64k_counters.table"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(each GPU's share would run the same kernels independently).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import attention_kl_divergence_online_amd as skl

    w = synth.get(args.workload)
    dev = "cuda"
    if args.fp8:
        # The fp8 line stands alone: the other workloads and the bf16
        # materialise-then-reduce comparison belong to the bf16 line.
        args.no_configs = True
        args.no_splitk = True
        args.materialised_heads = 0
    torch.cuda.init()
    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    q1, k1, q2, k2 = synth.make_inputs(w, device=dev)
    if args.fp8:
        q1, k1, q2, k2 = (synth.to_fp8(t) for t in (q1, k1, q2, k2))
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
        skl.streamkl_bwd_prepare(q1, k1, q2, k2, g, w.scale, w.causal, workspace=ws)
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
    # Device memory: everything the step touches is allocated above; the step
    # itself must add nothing (peak allocation during the timed steps minus
    # what is held before them).
    torch.cuda.reset_peak_memory_stats()
    held = torch.cuda.memory_allocated()

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
    extra_bytes = torch.cuda.max_memory_allocated() - held
    nbytes = lambda *ts: sum(t.numel() * t.element_size() for t in ts)
    memory = {
        "inputs_bytes": nbytes(q1, k1, q2, k2, g),
        "outputs_bytes": nbytes(kl, l1, l2, *grads),
        "workspace_bytes": nbytes(ws),  # sigma, operand scales and their chunk maxima: O(B*H)
        "extra_during_step_bytes": extra_bytes,
        # P1 and P2 as full NQ x NK bf16 matrices, which the fused path never forms.
        "materialised_p_bytes": 2 * 2 * w.B * w.H * w.NQ * w.NK,
    }
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps
    samples = {"fwd": [], "bwd_prepare": [], "bwd_dk": [], "bwd_dq": []}
    for e in evs:
        for i, k in enumerate(samples):
            samples[k].append(e[i].elapsed_time(e[i + 1]))
    per = {k: sum(v) / len(v) for k, v in samples.items()}
    fwd_ms = per["fwd"]
    bwd_ms = per["bwd_prepare"] + per["bwd_dk"] + per["bwd_dq"]

    pairs = w.visible_pairs()
    fwd_flop = 4 * w.D * pairs
    bwd_flop = 12 * w.D * pairs
    tflops = (fwd_flop + bwd_flop) / (ms_step * 1e-3) / 1e12

    # Roofline of the longest kernel.  Algorithmic flop per launch: forward 4*D
    # per visible pair; the backward 12*D per pair (both logit tiles, 4*D, and
    # the four gradient products, 8*D), counted as 6*D for each of its two
    # passes.  Each pass executes 8*D per pair (it recomputes both logit tiles
    # and forms two of the four gradient products); that rate is reported
    # beside the algorithmic one, never in its place.
    kern_flop = {"fwd": fwd_flop, "bwd_dk": 6 * w.D * pairs, "bwd_dq": 6 * w.D * pairs}
    exec_flop = {"fwd": fwd_flop, "bwd_dk": 8 * w.D * pairs, "bwd_dq": 8 * w.D * pairs}
    dom = max(kern_flop, key=lambda k: per[k])
    achieved = kern_flop[dom] / (per[dom] * 1e-3) / 1e12
    executed = exec_flop[dom] / (per[dom] * 1e-3) / 1e12
    kernel_names = {"fwd": "fwd2_kernel<128,unsplit,8 waves,128-key tiles,bf16>",
                    "bwd_dk": "bwd4_kernel<128,keys resident,both,bf16>",
                    "bwd_dq": "bwd4_kernel<128,queries resident,both,bf16>"}
    if args.fp8:
        kernel_names = {"fwd": "fwd2_kernel<128,unsplit,12 waves,128-key tiles,fp8>",
                        "bwd_dk": "bwd4_kernel<128,keys resident,both,fp8>",
                        "bwd_dq": "bwd4_kernel<128,queries resident,both,fp8>"}

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
        "dtype": "fp8_e4m3" if args.fp8 else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "NQ": w.NQ, "NK": w.NK, "D": w.D,
                   "causal": w.causal, "inputs": "fp8_e4m3" if args.fp8 else "bf16", "accumulate": "fp32"},
        "fwd_ms": round(fwd_ms, 3),
        "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
        "bwd_ms": round(bwd_ms, 3),
        "bwd_tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
        "kernel_ms": {k: round(v, 3) for k, v in per.items()},
        "kernel_tflops": {k: round(kern_flop[k] / (per[k] * 1e-3) / 1e12, 2) for k in kern_flop},
        "kernel_ms_median": {k: round(statistics.median(v), 3) for k, v in samples.items()},
        "kernel_ms_min": {k: round(min(v), 3) for k, v in samples.items()},
        "wall_s_timed": round(wall, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": kernel_names[dom],
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if args.fp8 else recorded_traffic(dom),
            "flop_per_launch": kern_flop[dom],
            "flop_rule": "algorithmic: 4*D per visible pair (forward), 6*D per pair per backward pass "
                         "(12*D for the whole backward)",
            "executed": {"flop_per_launch": exec_flop[dom], "tflops": round(executed, 2),
                         "frac": round(executed / PEAK_BF16_TFLOPS, 4),
                         "flop_rule": "8*D per pair per backward pass (both logit tiles recomputed in each)"},
        },
        "memory": memory,
    }

    # Sustained matrix rate under a full load (register operands only), set
    # beside the published peak the roofline fraction is taken against.
    progress(f"timed steps done: {ms_step:.3f} ms per step")
    out["roofline"]["measured_peak"] = round(mfma_probe(skl, torch), 1)

    if not args.no_splitk:
        out["splitk"] = splitk_bench(skl, synth, torch, args)
        progress("split-K forward done")

    if not args.no_configs:
        # Every workload of the metric in one line: algorithmic TFLOP/s and the
        # fraction of the matrix peak for the inputs' type (bf16 / fp32).
        cfgs = {"C4": {"workload": w.name, "fwd_ms": out["fwd_ms"], "bwd_ms": out["bwd_ms"],
                       "fwd_tflops": out["fwd_tflops"], "bwd_tflops": out["bwd_tflops"], "step_tflops": out["value"],
                       "fwd_frac": round(out["fwd_tflops"] / PEAK_BF16_TFLOPS, 4),
                       "bwd_frac": round(out["bwd_tflops"] / PEAK_BF16_TFLOPS, 4),
                       "step_frac": round(out["value"] / PEAK_BF16_TFLOPS, 4)}}
        for tag, name in CONFIGS:
            cfgs[tag] = config_bench(skl, synth, torch, args, name)
            progress(f"{tag} ({name}) done")
        if "splitk" in out:
            sk = dict(out["splitk"])
            sk["fwd_frac"] = round(sk["tflops"] / PEAK_BF16_TFLOPS, 4)
            cfgs["C5_fwd"] = sk
        out["configs"] = {k: cfgs[k] for k in ("C1", "C2", "C3", "C4", "C5_fwd", "C5_bwd") if k in cfgs}

    if not args.no_configs:
        # The same workload with e4m3 inputs (the fp8 path), beside the bf16 line.
        out["fp8"] = config_bench(skl, synth, torch, args, w.name, fp8=True)
        progress("fp8 step done")
        out["fused_vs_split"] = {n: fused_vs_split(skl, synth, torch, args, n)
                                 for n in ("shortq16_bwd_64k", "decode_128k", "shortq128_bwd_64k", "shortq_bwd_64k")}
        progress("fused vs split done")

    if args.other_configs:
        out["other_configs"] = {n: config_bench(skl, synth, torch, args, n)
                                for n in ("shortq_bwd_64k", "causal_16k_d64", "causal_4k_fp32")}
        out["other_configs"]["decode_128k"] = splitk_bench(skl, synth, torch, args, "decode_128k")
        out["other_configs"]["varlen_mix"] = varlen_bench(skl, synth, torch, args, "varlen_mix")
        out["other_configs"]["varlen_short"] = varlen_bench(skl, synth, torch, args, "varlen_short")

    if args.materialised_heads > 0:
        mat = materialised_baseline(torch, w, q1, k1, q2, k2, g, kl, args.materialised_heads)
        progress("materialised baseline done")
        mat["fwd_speedup_fused"] = round(mat["fwd_ms"] / fwd_ms, 1)
        mat["fwd_bwd_speedup_fused"] = round(mat["fwd_bwd_ms"] / ms_step, 1)
        out["materialised_baseline"] = mat

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, q1, k1, q2, k2, args.cpu_seconds)
        progress("cpu baseline done")

    print(json.dumps(out), flush=True)


def materialised_rows(nk: int) -> int:
    """Query rows per block of the materialised baseline: at most 2^30 logits per matrix."""
    return max(1, (1 << 30) // max(1, nk))


def materialised_baseline(torch, w, q1, k1, q2, k2, g, kl_fused, heads: int):
    """PyTorch materialise-then-reduce on the GPU, head by head and in blocks
    of query rows (at most 2^30 logits per matrix): both fp32 logit matrices,
    log-softmax, KL = sum P1 (log P1 - log P2) per row, and its autograd
    backward to all four inputs.  Timed on `heads` (b, h) slices after one
    untimed slice and scaled to the whole batch; the whole problem's P1 and P2
    would not fit in device memory.  Context for the fused path, not a
    reference: parity is held against the oracle."""
    ev = lambda: torch.cuda.Event(enable_timing=True)
    NQ, NK = w.NQ, w.NK
    off = NK - NQ
    rows = min(NQ, materialised_rows(NK))

    def one(b, h, grad):
        ins = [t[b, h].float().requires_grad_(grad) for t in (q1, k1, q2, k2)]
        a1, c1, a2, c2 = ins
        c1t, c2t = c1.t().contiguous(), c2.t().contiguous()
        parts = []
        for r0 in range(0, NQ, rows):
            r1 = min(NQ, r0 + rows)
            with torch.set_grad_enabled(grad):
                s1 = (a1[r0:r1] @ c1t) * w.scale
                s2 = (a2[r0:r1] @ c2t) * w.scale
                if w.causal:  # a large finite fill keeps 0 * (l1 - l2) at 0 on masked keys
                    mask = (torch.arange(NK, device=s1.device)[None, :] >
                            torch.arange(r0, r1, device=s1.device)[:, None] + off)
                    s1 = s1.masked_fill(mask, -1e30)
                    s2 = s2.masked_fill(mask, -1e30)
                l1 = torch.log_softmax(s1, dim=-1)
                l2 = torch.log_softmax(s2, dim=-1)
                del s1, s2
                kl = (l1.exp() * (l1 - l2)).sum(dim=-1)
                del l1, l2
                if grad:
                    (g[b, h, r0:r1] * kl).sum().backward()
            parts.append(kl.detach())
        return torch.cat(parts)

    units = [(u // w.H, u % w.H) for u in range(w.B * w.H)]
    timed = units[:heads]
    one(*units[-1], False)
    one(*units[-1], True)
    torch.cuda.synchronize()
    worst = 0.0
    res = {}
    for grad in (False, True):
        e0, e1 = ev(), ev()
        e0.record()
        outs = [one(b, h, grad) for b, h in timed]
        e1.record()
        torch.cuda.synchronize()
        res["fwd_bwd" if grad else "fwd"] = e0.elapsed_time(e1) * len(units) / len(timed)
        for (b, h), o in zip(timed, outs):
            ref = kl_fused[b, h]
            worst = max(worst, ((o - ref).abs().max() / ref.abs().max().clamp_min(1e-30)).item())
        del outs
    torch.cuda.empty_cache()
    return {"kind": "pytorch materialise-then-reduce (fp32 logits from the bf16 inputs, log_softmax, "
                    "autograd backward), head by head in blocks of query rows",
            "heads_timed": len(timed), "scaled_to_heads": len(units),
            "fwd_ms": round(res["fwd"], 1), "fwd_bwd_ms": round(res["fwd_bwd"], 1),
            "kl_max_rel_diff_vs_fused": float(f"{worst:.3g}"),
            "peak_alloc_bytes": torch.cuda.max_memory_allocated()}


def mfma_probe(skl, torch, iters: int = 100000, workgroups: int = 1024) -> float:
    """TFLOP/s of the library's bf16 matrix-rate probe: four waves per SIMD on
    every CU, each wave four independent 32x32x16 product chains, best of
    three runs after one warm-up."""
    sink = torch.empty(4 * workgroups, dtype=torch.float32, device="cuda")
    skl.streamkl_probe_mfma_bf16(iters, workgroups, sink)
    best = float("inf")
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        skl.streamkl_probe_mfma_bf16(iters, workgroups, sink)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return workgroups * 4 * iters * 4 * 32768 / (best * 1e-3) / 1e12


def config_bench(skl, synth, torch, args, name, fp8=False):
    """Forward (split-K when the workload sets a split count) and full backward
    (prepare + both passes) of one workload; HIP-event ms per step.  With
    `fp8` the workload's inputs are rounded to e4m3 first (the fp8 path)."""
    w = synth.get(name)
    q1, k1, q2, k2 = synth.make_inputs(w, device="cuda")
    if fp8:
        q1, k1, q2, k2 = (synth.to_fp8(t) for t in (q1, k1, q2, k2))
    g = synth.upstream_grad(w, "cuda")
    kl, l1, l2 = (torch.empty((w.B, w.H, w.NQ), dtype=torch.float32, device="cuda") for _ in range(3))
    grads = tuple(torch.empty_like(t, dtype=torch.float32) for t in (q1, k1, q2, k2))
    ws = torch.empty(max(16, skl.bwd_workspace_size(q1, k1, w.scale, w.causal)), dtype=torch.uint8, device="cuda")
    wsk = None
    if w.splits > 1:
        wsk = torch.empty(skl.fwd_splitk_workspace_size(q1, k1, w.splits, w.scale, w.causal), dtype=torch.uint8,
                          device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd_ms = bwd_ms = 0.0
    for it in range(args.warmup + args.steps):
        ev[0].record()
        if wsk is None:
            skl.streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal, out=(kl, l1, l2))
        else:
            skl.streamkl_fwd_splitk(q1, k1, q2, k2, w.splits, w.scale, w.causal, workspace=wsk, out=(kl, l1, l2))
        ev[1].record()
        skl.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal, workspace=ws, out=grads)
        ev[2].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            fwd_ms += ev[0].elapsed_time(ev[1]) / args.steps
            bwd_ms += ev[1].elapsed_time(ev[2]) / args.steps
    pairs = w.visible_pairs()
    peak = PEAK_FP32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS
    fwd_t = 4 * w.D * pairs / (fwd_ms * 1e-3) / 1e12
    bwd_t = 12 * w.D * pairs / (bwd_ms * 1e-3) / 1e12
    step_t = 16 * w.D * pairs / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
    res = {"workload": w.name, "fwd_splits": w.splits, "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
           "fwd_tflops": round(fwd_t, 2), "bwd_tflops": round(bwd_t, 2), "step_tflops": round(step_t, 2),
           "peak_tflops": peak, "fwd_frac": round(fwd_t / peak, 4), "bwd_frac": round(bwd_t / peak, 4),
           "step_frac": round(step_t / peak, 4)}
    if fp8:
        # The forward's products and the backward's logits run at the fp8
        # matrix rate, the backward's gradient products (8*D of its 12*D per
        # pair) at the fp16 one; fractions stay against the bf16/fp16 peak,
        # with the forward's also against the fp8 peak.
        res["inputs"] = "fp8_e4m3"
        res["fwd_frac_fp8_peak"] = round(fwd_t / PEAK_FP8_TFLOPS, 4)
    del q1, k1, q2, k2, grads, ws, wsk
    torch.cuda.empty_cache()
    return res


def fused_vs_split(skl, synth, torch, args, name):
    """Backward of a short-query workload through the combined call (the fused
    single-visit pass where the query count allows, else the split passes)
    and through the step-wise calls (always the split passes: prepare, dK
    pass, dQ pass); HIP-event ms per backward and algorithmic TFLOP/s."""
    w = synth.get(name)
    q1, k1, q2, k2 = synth.make_inputs(w, device="cuda")
    g = synth.upstream_grad(w, "cuda")
    kl, l1, l2 = skl.streamkl_fwd_splitk(q1, k1, q2, k2, w.splits, w.scale, w.causal)
    grads = tuple(torch.empty_like(t, dtype=torch.float32) for t in (q1, k1, q2, k2))
    ws = torch.empty(max(16, skl.bwd_workspace_size(q1, k1, w.scale, w.causal)), dtype=torch.uint8, device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    comb = split = 0.0
    for it in range(args.warmup + args.steps):
        ev[0].record()
        skl.streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal, workspace=ws, out=grads)
        ev[1].record()
        skl.streamkl_bwd_prepare(q1, k1, q2, k2, g, w.scale, w.causal, workspace=ws)
        skl.streamkl_bwd_dk(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal, workspace=ws, out=(grads[1], grads[3]))
        skl.streamkl_bwd_dq(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal, workspace=ws, out=(grads[0], grads[2]))
        ev[2].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            comb += ev[0].elapsed_time(ev[1]) / args.steps
            split += ev[1].elapsed_time(ev[2]) / args.steps
    flop = 12 * w.D * w.visible_pairs()
    fused = w.dtype == "bf16" and w.NQ <= 128
    res = {"B": w.B, "H": w.H, "NQ": w.NQ, "NK": w.NK, "combined_path": "fused" if fused else "split",
           "combined_ms": round(comb, 3), "split_ms": round(split, 3),
           "combined_tflops": round(flop / (comb * 1e-3) / 1e12, 2), "split_tflops": round(flop / (split * 1e-3) / 1e12, 2),
           "split_over_combined": round(split / comb, 2),
           # fp32 key gradients written plus keys read once: the fused pass's HBM floor.
           "dk_write_plus_k_read_gb": round((2 * 4 + 2 * 2) * w.B * w.H * w.NK * w.D / 1e9, 2)}
    del q1, k1, q2, k2, grads, ws
    torch.cuda.empty_cache()
    return res


def varlen_bench(skl, synth, torch, args, name):
    """Forward and full backward of a packed variable-length batch; HIP-event ms per step."""
    pb = synth.PACKED[name]
    q1, k1, q2, k2 = synth.make_packed(pb, "cuda")
    cq, ck = pb.cu_q, pb.cu_k
    g = synth.packed_grad(pb, "cuda")
    out = tuple(torch.empty(q1.shape[:2], dtype=torch.float32, device="cuda") for _ in range(3))
    grads = tuple(torch.empty_like(t, dtype=torch.float32) for t in (q1, k1, q2, k2))
    ws = torch.empty(skl.bwd_varlen_workspace_size(q1, k1, cq, ck, pb.scale, pb.causal), dtype=torch.uint8,
                     device="cuda")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd_ms = bwd_ms = 0.0
    for it in range(args.warmup + args.steps):
        ev[0].record()
        skl.streamkl_fwd_varlen(q1, k1, q2, k2, cq, ck, pb.scale, pb.causal, out=out)
        ev[1].record()
        skl.streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, *out, g, pb.scale, pb.causal, workspace=ws, out=grads)
        ev[2].record()
        torch.cuda.synchronize()
        if it >= args.warmup:
            fwd_ms += ev[0].elapsed_time(ev[1]) / args.steps
            bwd_ms += ev[1].elapsed_time(ev[2]) / args.steps
    pairs = pb.visible_pairs()
    res = {"sequences": len(pb.lens_q), "rows": cq[-1], "fwd_ms": round(fwd_ms, 3), "bwd_ms": round(bwd_ms, 3),
           "fwd_tflops": round(4 * pb.D * pairs / (fwd_ms * 1e-3) / 1e12, 2),
           "bwd_tflops": round(12 * pb.D * pairs / (bwd_ms * 1e-3) / 1e12, 2),
           "step_tflops": round(16 * pb.D * pairs / ((fwd_ms + bwd_ms) * 1e-3) / 1e12, 2)}
    del q1, k1, q2, k2, grads, ws
    torch.cuda.empty_cache()
    return res


def splitk_bench(skl, synth, torch, args, name="splitk_512k"):
    """Split-K forward (splits from the workload); also the HBM rate of reading the keys once."""
    w = synth.get(name)
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
    key_bytes = 2 * w.B * w.H * w.NK * w.D * 2  # K1 and K2, bf16, read once
    res = {"workload": w.name, "splits": w.splits, "ms": round(ms, 3),
           "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
           "key_read_gbs": round(key_bytes / (ms * 1e-3) / 1e9, 1)}
    del q1, k1, q2, k2, ws
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
