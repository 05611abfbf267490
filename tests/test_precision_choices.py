"""Precision choices of the kernels, checked with the oracle on the CPU.

The bf16 path keeps its inputs in bf16 and accumulates in fp32.  Rounding the
inputs further, to fp8 (e4m3), would take the outputs outside the 2e-3
relative bound by itself, before any kernel error: this is why the matrix
cores' fp8 rate is not used for the logits.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import rel_err

pytestmark = pytest.mark.skipif(not hasattr(torch, "float8_e4m3fn"), reason="torch without float8 types")


def _inputs(N=512, D=128, noise=0.1, seed=3):
    g = torch.Generator().manual_seed(seed)
    q1 = torch.randn(N, D, generator=g)
    k1 = torch.randn(N, D, generator=g)
    q2 = q1 + noise * torch.randn(N, D, generator=g)
    k2 = k1 + noise * torch.randn(N, D, generator=g)
    return q1, k1, q2, k2


def _rounded(ts, dt):
    return [t.to(dt).to(torch.float64).numpy() for t in ts]


def test_fp8_inputs_break_the_bound_bf16_inputs_define():
    ts = _inputs()
    scale = 1.0 / np.sqrt(128)
    ref = oracle.fwd(*_rounded(ts, torch.bfloat16), scale, True)
    f8 = oracle.fwd(*_rounded(ts, torch.float8_e4m3fn), scale, True)
    errs = {name: rel_err(a, b) for name, a, b in zip(("kl", "lse1", "lse2"), f8, ref)}
    # fp8 rounding alone moves KL by tens of percent and the LSEs past 2e-3.
    assert errs["kl"] > 0.1, errs
    assert errs["lse1"] > 2e-3 and errs["lse2"] > 2e-3, errs
    # The rounding noise raises the mean KL (it adds variance to both logit sets).
    assert np.mean(f8[0]) > np.mean(ref[0])


def test_ds_in_bf16_breaks_the_bound_scaled_fp16_keeps_it():
    # The backward's gradient products take dS as a 16-bit operand.  dS comes from
    # autograd over the materialised definition (fp64, one head of 4096 rows, a peaky
    # teacher against an independent student), and only its rounding differs.
    N, D = 4096, 128
    g = torch.Generator().manual_seed(0)
    q1 = (torch.randn(N, D, generator=g, dtype=torch.float64) * 1.5).to(torch.bfloat16).double()
    k1 = (torch.randn(N, D, generator=g, dtype=torch.float64) * 1.5).to(torch.bfloat16).double()
    q2 = torch.randn(N, D, generator=g, dtype=torch.float64).to(torch.bfloat16).double()
    k2 = torch.randn(N, D, generator=g, dtype=torch.float64).to(torch.bfloat16).double()
    scale = 1.0 / np.sqrt(D)
    s1 = (scale * q1 @ k1.T).requires_grad_(True)
    s2 = (scale * q2 @ k2.T).requires_grad_(True)
    l1, l2 = torch.log_softmax(s1, -1), torch.log_softmax(s2, -1)
    kl = (l1.exp() * (l1 - l2)).sum(-1)
    gw = 1.0 / (32 * N)
    (gw * kl).sum().backward()
    for ds, k in ((s1.grad, k1), (s2.grad, k2)):
        dq = scale * ds @ k
        err = lambda r: ((scale * r @ k - dq).abs().max() / dq.abs().max()).item()
        bf16 = err(ds.float().to(torch.bfloat16).double())
        sigma = 2.0 ** 7 / gw  # |g| * sigma in [2^7, 2^8), as the kernels scale it
        fp16 = err((ds * sigma).float().to(torch.float16).double() / sigma)
        assert bf16 > 2e-3, bf16
        assert fp16 < 5e-4, fp16
