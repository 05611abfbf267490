"""Shared helpers for the GPU-vs-oracle parity tests.

Error measure: for an output tensor T of one (batch, head) slice,
    err = max |T_gpu - T_ref| / max |T_ref|
(per-element relative error is ill-posed where KL or an LSE is ~0, e.g. the
causal first row has KL = 0 exactly).  Bounds: 2e-3 for bf16 inputs with fp32
accumulation, 1e-5 for fp32 inputs.

Reported beside the gated figures, never gated: the largest per-row relative
KL error over rows whose reference KL is at least 1e-3 of the slice's largest
(`info_kl_row_rel`), and the largest absolute LSE error in nats
(`info_lse_abs`); keys starting with "info_" are logged, not bounded.
"""
from __future__ import annotations

import json
import math
import os
from typing import Dict, Iterable, List, Sequence

import numpy as np
import torch

import oracle

TOL = {"bf16": 2e-3, "fp32": 1e-5}


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(gpu - ref))
    if not np.all(np.isfinite(gpu)):
        return math.inf
    if den == 0.0:
        return float(num)
    return float(num / den)


def head(t: torch.Tensor, b: int, h: int) -> np.ndarray:
    return t[b, h].detach().to("cpu", torch.float64).numpy()


def sample_rows(n: int, count: int, seed: int, tile: int = 256) -> List[int]:
    """First and last rows, rows around tile edges, and random rows (all rows if count >= n)."""
    if count >= n:
        return list(range(n))
    rng = np.random.default_rng(seed)
    rows = {0, 1, n - 1, n - 2}
    for e in (tile - 1, tile, 2 * tile - 1, n // 2):
        if 0 <= e < n:
            rows.add(e)
    rows.update(rng.integers(0, n, size=max(0, count - len(rows))).tolist())
    return sorted(r for r in rows if 0 <= r < n)


def compare_forward(q1, k1, q2, k2, scale, causal, kl, lse1, lse2,
                    heads: Iterable, rows: Sequence[int] = None) -> Dict[str, float]:
    """Worst err over the given heads for KL, LSE1, LSE2 (all rows or `rows`)."""
    worst = {"kl": 0.0, "lse1": 0.0, "lse2": 0.0, "info_kl_row_rel": 0.0, "info_lse_abs": 0.0}
    for b, h in heads:
        rk, r1, r2 = oracle.fwd(head(q1, b, h), head(k1, b, h), head(q2, b, h), head(k2, b, h),
                                scale, causal, rows=rows)
        sel = slice(None) if rows is None else list(rows)
        for name, gt, rt in (("kl", kl, rk), ("lse1", lse1, r1), ("lse2", lse2, r2)):
            g = gt[b, h].detach().cpu().double().numpy()[sel]
            worst[name] = max(worst[name], rel_err(g, rt))
            rt = np.asarray(rt, dtype=np.float64)
            if name == "kl":
                worst["info_kl_row_rel"] = max(worst["info_kl_row_rel"], row_rel_err(g, rt))
            else:
                worst["info_lse_abs"] = max(worst["info_lse_abs"], float(np.max(np.abs(g - rt), initial=0.0)))
    return worst


def row_rel_err(gpu, ref, floor: float = 1e-3) -> float:
    """Largest |gpu - ref| / |ref| over the rows whose |ref| is at least `floor`
    times the largest |ref| (0 when no row qualifies)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    top = np.max(np.abs(ref), initial=0.0)
    keep = np.abs(ref) >= floor * top
    if top == 0.0 or not np.any(keep):
        return 0.0
    return float(np.max(np.abs(gpu[keep] - ref[keep]) / np.abs(ref[keep])))


def compare_backward(q1, k1, q2, k2, scale, causal, g, grads, heads: Iterable,
                     rows: Sequence[int] = None, check_dk: bool = True) -> Dict[str, float]:
    """Worst err of (dq1, dk1, dq2, dk2) against the oracle.

    With `rows`, dQ is compared on those rows and dK (if check_dk) against the
    contribution of those rows only -- valid when g is zero on every other row."""
    dq1, dk1, dq2, dk2 = grads
    worst = {"dq1": 0.0, "dk1": 0.0, "dq2": 0.0, "dk2": 0.0}
    for b, h in heads:
        gh = g[b, h].detach().cpu().double().numpy()
        r = np.arange(gh.size) if rows is None else np.asarray(rows)
        out = oracle.bwd(head(q1, b, h), head(k1, b, h), head(q2, b, h), head(k2, b, h), scale, causal,
                         gh[r], rows=r)
        for name, gt in (("dq1", dq1), ("dq2", dq2)):
            worst[name] = max(worst[name], rel_err(gt[b, h].detach().cpu().double().numpy()[r], out[name]))
        if check_dk:
            for name, gt in (("dk1", dk1), ("dk2", dk2)):
                worst[name] = max(worst[name], rel_err(gt[b, h].detach().cpu().double().numpy(), out[name]))
    return worst


def assert_within(errs: Dict[str, float], tol: float, what: str) -> None:
    log = os.environ.get("PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(json.dumps({"case": what, "tol": tol, "errs": errs}) + "\n")
    info = {k: v for k, v in errs.items() if k.startswith("info_")}
    if info:
        print(f"{what}: " + ", ".join(f"{k[5:]} {v:.3g}" for k, v in info.items()), flush=True)
    bad = {k: v for k, v in errs.items() if not k.startswith("info_") and not (v <= tol)}
    assert not bad, f"{what}: err above {tol}: {bad} (all: {errs})"
