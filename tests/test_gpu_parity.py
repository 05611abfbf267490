"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes span several tiles with ragged tails in both N_Q and N_K and are
compared element by element.  The full-size workloads (causal 4K, non-causal
16K, causal 64K, split-K 512K keys, 128K-key backward) run in the launch
configuration the benchmark times and are compared on sampled rows the oracle
computes one by one; key gradients at full size are compared in full with an
upstream gradient that is nonzero only on the sampled rows (dK is linear in g),
plus the any-size invariant sum_j dK[j] = 0.
"""
import math

import numpy as np
import pytest
import torch

import synth
from attention_kl_divergence_online_amd import (StreamKLError, attention_kl, streamkl_bwd, streamkl_fwd,
                                                streamkl_fwd_splitk)
from parity_util import TOL, assert_within, compare_backward, compare_forward, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _rand(B, H, NQ, NK, D, dtype, seed, noise=0.3, std=1.0):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q1 = torch.randn(B, H, NQ, D, generator=g) * std
    k1 = torch.randn(B, H, NK, D, generator=g) * std
    q2 = q1 + noise * torch.randn(B, H, NQ, D, generator=g)
    k2 = k1 + noise * torch.randn(B, H, NK, D, generator=g)
    return [t.to(dtype).to(DEV).contiguous() for t in (q1, k1, q2, k2)]


def _heads(B, H):
    return [(b, h) for b in range(B) for h in range(H)]


def test_device_present():
    assert torch.cuda.is_available(), "no HIP device visible"


def test_tiny_fp32_workload_full():
    w = synth.get("tiny_fp32")
    q1, k1, q2, k2 = (t.to(DEV) for t in synth.make_inputs(w))
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal)
    g = synth.upstream_grad(w, DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal)
    torch.cuda.synchronize()
    heads = _heads(w.B, w.H)
    assert_within(compare_forward(q1, k1, q2, k2, w.scale, w.causal, kl, l1, l2, heads), TOL["fp32"], "fwd")
    assert_within(compare_backward(q1, k1, q2, k2, w.scale, w.causal, g, grads, heads), TOL["fp32"], "bwd")


SMALL = [
    # B, H, NQ, NK, D, causal
    (1, 2, 300, 517, 128, False),
    (1, 2, 300, 517, 128, True),
    (2, 1, 700, 700, 128, True),
    (1, 3, 129, 1000, 64, False),
    (1, 2, 257, 333, 64, True),
    (1, 1, 1, 37, 128, False),
    (1, 1, 1, 1, 128, False),
    (1, 1, 5, 5, 128, True),
    (1, 2, 64, 4100, 128, False),
    (2, 1, 16, 77, 64, True),      # bf16: 16x16-product forward shape at its 16-query limit
    (1, 2, 32, 200, 64, True),     # bf16: one-wave forward shape at its 32-query limit
    (1, 1, 33, 97, 128, False),    # bf16: one query past it (8-wave shape, one live wave)
    (3, 4, 300, 520, 128, True),   # 12 heads: causal backward tiles dealt round the XCDs, forward in runs
    (2, 4, 520, 520, 64, True),    # 8 heads: whole heads per XCD
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,H,NQ,NK,D,causal", SMALL)
def test_small_shapes_full(dtype, B, H, NQ, NK, D, causal):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"case {dtype} B={B} H={H} NQ={NQ} NK={NK} D={D} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, tdt, seed=NQ * 7 + NK + D)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    gen = torch.Generator(device="cpu").manual_seed(3)
    g = torch.rand(B, H, NQ, generator=gen).mul_(2).sub_(0.5).to(DEV)  # mixed signs
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    heads = _heads(B, H)
    case = f"{dtype} B{B} H{H} NQ{NQ} NK{NK} D{D} causal={causal}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL[dtype], f"fwd {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, grads, heads), TOL[dtype], f"bwd {case}")


PEAKED = [
    # D, scale, causal: raw logit ranges of about 130 and 270 per row, row KL up to
    # about 100 and 190 (teacher and student independent), so nearly one-hot rows,
    # rescaling by large max jumps, and dS1 terms with large log-ratios.
    (64, 2.0, False),
    (64, 4.0, True),
    (128, 2.0, True),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,scale,causal", PEAKED)
def test_peaked_rows_large_kl(dtype, D, scale, causal):
    B, H, NQ, NK = 1, 2, 200, 333
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"peaked {dtype} D={D} scale={scale} causal={causal}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(int(D + 10 * scale + causal))
    q1, k1, q2, k2 = (torch.randn(B, H, n, D, generator=gen).to(tdt).to(DEV).contiguous()
                      for n in (NQ, NK, NQ, NK))
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    g = (torch.rand(B, H, NQ, generator=gen) - 0.3).to(DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    kls, l1s, l2s = streamkl_fwd_splitk(q1, k1, q2, k2, 3, scale, causal)
    torch.cuda.synchronize()
    assert kl.max().item() > 30.0  # the regime this case is for
    heads = _heads(B, H)
    case = f"peaked {dtype} D{D} scale={scale} causal={causal}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL[dtype], f"fwd {case}")
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kls, l1s, l2s, heads), TOL[dtype],
                  f"split fwd {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, grads, heads), TOL[dtype], f"bwd {case}")
    for t in grads:
        assert torch.isfinite(t).all()


@pytest.mark.parametrize("slope", [0.2, -0.2])
@pytest.mark.parametrize("causal,NQ,NK", [(False, 260, 1100), (True, 260, 1100), (True, 4200, 4300)])
def test_monotone_logits_held_maxima(slope, causal, NQ, NK):
    # Keys along one direction with a steady rise (or fall) along the key
    # index: each raw logit differs from the previous key's by about
    # 2.3 * slope / 0.2, so with rising logits the maxima a lane holds go
    # stale by far more than 2^24 within a few 32-key blocks (the forward
    # folds those blocks again exactly), and with falling logits the first
    # block holds the maxima and later terms underflow.  Causal problems of
    # more than 4096 queries run the eight-wave, 128-key-tile forward shape
    # (its diagonal masking and refold), shorter ones the four-wave shape.
    B, H, D = 1, 2 if NQ < 1000 else 1, 128
    print(f"monotone logits slope={slope} causal={causal} NQ={NQ} NK={NK}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(int(100 * slope) + causal)
    u = torch.randn(D, generator=gen)
    u = u / u.norm()
    j = torch.arange(NK, dtype=torch.float32)[:, None]
    q1 = 11.3 * u + 0.5 * torch.randn(B, H, NQ, D, generator=gen)
    q2 = 11.3 * u + 0.5 * torch.randn(B, H, NQ, D, generator=gen)
    k1 = slope * j * u + 0.3 * torch.randn(B, H, NK, D, generator=gen)
    k2 = 0.8 * slope * j * u + 0.3 * torch.randn(B, H, NK, D, generator=gen)
    q1, k1, q2, k2 = (t.to(torch.bfloat16).to(DEV).contiguous() for t in (q1, k1, q2, k2))
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    kls, l1s, l2s = streamkl_fwd_splitk(q1, k1, q2, k2, 3, scale, causal)
    torch.cuda.synchronize()
    heads = _heads(B, H)
    case = f"monotone slope={slope} causal={causal}"
    assert kl.max().item() > 0.05  # teacher and student spread differently
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"], f"fwd {case}")
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kls, l1s, l2s, heads), TOL["bf16"],
                  f"split fwd {case}")


@pytest.mark.parametrize("offset", [0.0, 1000.0, 1400.0])
@pytest.mark.parametrize("causal", [False, True])
def test_teacher_maxima_far_above_the_students(offset, causal):
    # The teacher's keys share a component along its queries' direction, so
    # its logits carry a common offset of about `offset` raw units (0.127 *
    # offset in log2 units at D = 128) on top of a spread of about 3% of it:
    # its held maxima sit that far above the student's.  The forward's
    # steady state takes both distributions' terms against the mean of the
    # two maxima while they are at most 160 log2 units apart (offset 1000)
    # and folds every block exactly beyond that (offset 1400).
    B, H, NQ, NK, D = 1, 2, 700, 1500, 128
    print(f"far-apart maxima offset={offset} causal={causal}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(int(offset) + causal)
    u = torch.randn(D, generator=gen)
    u = u / u.norm()
    q1 = (offset / 10.0) * u + 0.7 * torch.randn(B, H, NQ, D, generator=gen)
    k1 = 10.0 * u + 0.3 * torch.randn(B, H, NK, D, generator=gen)
    q2 = torch.randn(B, H, NQ, D, generator=gen)
    k2 = torch.randn(B, H, NK, D, generator=gen)
    q1, k1, q2, k2 = (t.to(torch.bfloat16).to(DEV).contiguous() for t in (q1, k1, q2, k2))
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    kls, l1s, l2s = streamkl_fwd_splitk(q1, k1, q2, k2, 3, scale, causal)
    torch.cuda.synchronize()
    heads = _heads(B, H)
    case = f"far-apart maxima offset={offset} causal={causal}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"], f"fwd {case}")
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kls, l1s, l2s, heads), TOL["bf16"],
                  f"split fwd {case}")


@pytest.mark.parametrize("NQ,NK", [(4160, 4160), (4100, 4357)])
def test_causal_eight_wave_shape_all_rows(NQ, NK):
    # Causal bf16 problems just past 4096 queries take the forward's eight-wave
    # shape (256 queries over 128-key tiles) that the 64K workload runs: every
    # row of the forward and every gradient against the oracle, with a ragged
    # last query tile and, for NQ < NK, a diagonal offset.
    B, H, D = 1, 1, 128
    print(f"eight-wave causal NQ={NQ} NK={NK}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, torch.bfloat16, seed=NQ + NK, noise=0.1)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, True)
    gen = torch.Generator(device="cpu").manual_seed(NQ)
    g = (torch.rand(B, H, NQ, generator=gen) - 0.3).to(DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, True)
    torch.cuda.synchronize()
    heads = _heads(B, H)
    case = f"eight-wave causal NQ{NQ} NK{NK}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, True, kl, l1, l2, heads), TOL["bf16"], f"fwd {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, True, g, grads, heads), TOL["bf16"], f"bwd {case}")


def test_backward_steps_equal_combined_call():
    from attention_kl_divergence_online_amd import streamkl_bwd_dk, streamkl_bwd_dq, streamkl_bwd_prepare
    q1, k1, q2, k2 = _rand(2, 2, 300, 400, 128, torch.bfloat16, seed=12)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, None, True)
    g = torch.rand(2, 2, 300, device=DEV) * 1e-3
    full = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True)
    ws = streamkl_bwd_prepare(q1, k1, q2, k2, g, None, True)
    dk1, dk2 = streamkl_bwd_dk(q1, k1, q2, k2, kl, l1, l2, g, None, True, workspace=ws)
    dq1, dq2 = streamkl_bwd_dq(q1, k1, q2, k2, kl, l1, l2, g, None, True, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip((dq1, dk1, dq2, dk2), full):
        assert torch.equal(a, b)


@pytest.mark.parametrize("splits", [2, 3, 7, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_splitk_small(splits, causal, dtype):
    # 1000 keys are 8 chunk tiles of 128: at 16 splits the last 8 chunks are empty.
    B, H, NQ, NK, D = 1, 2, 300, 1000, 128
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    print(f"split-K {dtype} splits={splits} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, tdt, seed=11 + splits)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd_splitk(q1, k1, q2, k2, splits, scale, causal)
    ukl, ul1, ul2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    torch.cuda.synchronize()
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, _heads(B, H)), TOL[dtype],
                  f"split {dtype} {splits}")
    for a, b in ((kl, ukl), (l1, ul1), (l2, ul2)):
        d = (a - b).abs().max().item() / max(b.abs().max().item(), 1e-30)
        assert d <= 1e-4, d  # both sides are also held to the oracle bound above


@pytest.mark.parametrize("NQ", [1, 16])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_splitk(NQ, causal, D):
    # Few queries against a long key range: the decode use of the split-K forward.
    B, H, NK = 2, 2, 5000
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, torch.bfloat16, seed=21 + NQ)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd_splitk(q1, k1, q2, k2, 16, scale, causal)
    torch.cuda.synchronize()
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, _heads(B, H)), TOL["bf16"],
                  f"decode NQ={NQ} causal={causal} D={D}")


def test_identical_teacher_student_is_zero_to_rounding():
    """KL(P || P) = 0 and its gradients vanish.  The forward forms the
    student's logits as the teacher's minus the student's products in one
    accumulation chain, so identical inputs leave a rounding residue of
    order 2^-24 of the logits (|x| <~ 40 here) in x1 - x2: KL, LSE2 - LSE1
    and the gradients are that small, not exactly zero."""
    q1, k1, _, _ = _rand(1, 2, 300, 300, 128, torch.bfloat16, seed=5)
    for causal in (False, True):
        kl, l1, l2 = streamkl_fwd(q1, k1, q1, k1, None, causal)
        g = torch.ones(1, 2, 300, device=DEV)
        grads = streamkl_bwd(q1, k1, q1, k1, kl, l1, l2, g, None, causal)
        torch.cuda.synchronize()
        worst = [kl.abs().max().item(), (l1 - l2).abs().max().item()] + [t.abs().max().item() for t in grads]
        print("identical inputs: |KL|, |LSE1 - LSE2|, |dQ1|, |dK1|, |dQ2|, |dK2| max", worst)
        assert worst[0] <= 2e-5 and worst[1] <= 2e-5
        assert max(worst[2:]) <= 2e-6


def test_zero_queries_uniform_rows():
    B, H, NQ, NK, D = 1, 1, 200, 300, 128
    _, k1, _, k2 = _rand(B, H, NQ, NK, D, torch.bfloat16, seed=6)
    z = torch.zeros(B, H, NQ, D, dtype=torch.bfloat16, device=DEV)
    for causal in (False, True):
        kl, l1, l2 = streamkl_fwd(z, k1, z, k2, None, causal)
        torch.cuda.synchronize()
        n = torch.arange(NQ, device=DEV) + (NK - NQ) + 1 if causal else torch.full((NQ,), NK, device=DEV)
        assert kl.abs().max().item() <= 1e-6
        torch.testing.assert_close(l1[0, 0], n.double().log().float(), rtol=2e-7, atol=2e-6)


def test_bitwise_repeatable():
    q1, k1, q2, k2 = _rand(1, 4, 700, 900, 128, torch.bfloat16, seed=7)
    g = torch.full((1, 4, 700), 1e-3, device=DEV)
    outs = []
    for _ in range(2):
        kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, None, True)
        sk = streamkl_fwd_splitk(q1, k1, q2, k2, 5, None, True)
        grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True)
        outs.append([t.clone() for t in (kl, l1, l2, *sk, *grads)])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_gradient_pairs_can_be_skipped():
    q1, k1, q2, k2 = _rand(1, 2, 200, 300, 128, torch.bfloat16, seed=8)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, None, False)
    g = torch.full((1, 2, 200), 0.01, device=DEV)
    full = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g)
    t_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, student=False)
    s_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, teacher=False)
    torch.cuda.synchronize()
    assert t_only[2] is None and s_only[0] is None
    assert torch.equal(t_only[0], full[0]) and torch.equal(t_only[1], full[1])
    assert torch.equal(s_only[2], full[2]) and torch.equal(s_only[3], full[3])


@pytest.mark.parametrize("D", [64, 128])
def test_single_configuration_passes_match_oracle(D):
    # Teacher-only (Configuration 2) and student-only (Configuration 1) passes
    # form only the dS they need; causal, NQ < NK, signed g.
    q1, k1, q2, k2 = _rand(1, 2, 300, 517, D, torch.bfloat16, seed=12)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, None, True)
    g = (torch.rand((1, 2, 300), generator=torch.Generator().manual_seed(13)) - 0.4).to(DEV)
    full = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True)
    t_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True, student=False)
    s_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True, teacher=False)
    torch.cuda.synchronize()
    for a, b in ((t_only[0], full[0]), (t_only[1], full[1]), (s_only[2], full[2]), (s_only[3], full[3])):
        assert torch.equal(a, b)
    scale = 1.0 / math.sqrt(D)
    grads = (t_only[0], t_only[1], s_only[2], s_only[3])
    errs = compare_backward(q1, k1, q2, k2, scale, True, g, grads, heads=[(0, 0), (0, 1)])
    assert_within(errs, TOL["bf16"], f"single-configuration passes D={D}")


def test_workspace_without_split_partials_runs_dq_unsplit():
    # Any workspace from the minimum (sigma, operand scales, chunk maxima) up
    # is accepted; below the full size the query pass runs unsplit instead of
    # over key chunks.  dK is bitwise the same, dQ equal up to the fp32
    # summation order of the chunk partials, and both sides meet the oracle.
    from attention_kl_divergence_online_amd import bwd_workspace_size, bwd_workspace_size_min
    q1, k1, q2, k2 = _rand(2, 3, 200, 333, 128, torch.bfloat16, seed=14)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, None, True)
    g = (torch.rand((2, 3, 200), generator=torch.Generator().manual_seed(15)) - 0.3).to(DEV)
    full = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True)
    lo, hi = bwd_workspace_size_min(q1, k1, None, True), bwd_workspace_size(q1, k1, None, True)
    assert 0 < lo < hi
    for nbytes in (lo, (lo + hi) // 2, hi - 16):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        got = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, None, True, workspace=ws)
        torch.cuda.synchronize()
        for i in (1, 3):
            assert torch.equal(got[i], full[i]), nbytes
        for i in (0, 2):
            d = (got[i] - full[i]).abs().max().item() / full[i].abs().max().item()
            assert d <= 1e-5, (nbytes, i, d)
    errs = compare_backward(q1, k1, q2, k2, 1.0 / math.sqrt(128), True, g, got, heads=_heads(2, 3))
    assert_within(errs, TOL["bf16"], "unsplit query pass")


# Inputs far from unit magnitude: the fp16 operands of the gradient products
# are scaled per (batch, head, tensor) by a power of two, so entries past the
# fp16 range (65504) or deep in its subnormals give finite, accurate gradients.
# Each case keeps the logits of the unscaled problem (Q and K scaled
# inversely, or `scale` compensating), so KL and LSE are those of a plain
# problem while dQ and dK scale with 1/k and 1/q.
SCALED = [
    # q factor, k factor, logit-scale factor, D, causal
    (2.0 ** 10, 2.0 ** -10, 1.0, 128, True),
    (2.0 ** 14, 2.0 ** -14, 1.0, 128, False),
    (2.0 ** -12, 2.0 ** -12, 2.0 ** 24, 64, True),
    (2.0 ** -16, 2.0 ** 16, 1.0, 64, False),
]


@pytest.mark.parametrize("fq,fk,fs,D,causal", SCALED)
def test_scaled_inputs_keep_fp16_operands_in_range(fq, fk, fs, D, causal):
    B, H, NQ, NK = 1, 2, 300, 517
    print(f"scaled inputs q*{fq} k*{fk} scale*{fs} D={D} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, torch.float32, seed=int(D + 7 * causal), noise=0.2)
    q1, q2 = (t * fq for t in (q1, q2))
    k1, k2 = (t * fk for t in (k1, k2))
    q1, k1, q2, k2 = (t.to(torch.bfloat16).contiguous() for t in (q1, k1, q2, k2))
    scale = fs / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    g = (torch.rand((B, H, NQ), generator=torch.Generator().manual_seed(D)) - 0.3).to(DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t).all()
    heads = _heads(B, H)
    case = f"scaled q*{fq} k*{fk} D{D} causal={causal}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"], f"fwd {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, grads, heads), TOL["bf16"], f"bwd {case}")


def test_no_device_memory_beyond_the_callers_buffers():
    # The library allocates nothing: with inputs, outputs and workspaces allocated
    # up front, the calls raise neither torch's peak allocation nor the device's
    # used memory (after one warm-up call, which lets the runtime set up).
    from attention_kl_divergence_online_amd import (bwd_workspace_size, fwd_splitk_workspace_size,
                                                    streamkl_fwd_varlen, streamkl_bwd_varlen,
                                                    bwd_varlen_workspace_size)
    B, H, N, D = 2, 8, 4096, 128
    print(f"memory B={B} H={H} N={N}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, N, N, D, torch.bfloat16, seed=17)
    outs = tuple(torch.empty(B, H, N, device=DEV) for _ in range(3))
    g = torch.full((B, H, N), 1e-3, device=DEV)
    grads = tuple(torch.empty(B, H, N, D, device=DEV) for _ in range(4))
    ws = torch.empty(bwd_workspace_size(q1, k1, None, True), dtype=torch.uint8, device=DEV)
    splits = 8
    wsk = torch.empty(fwd_splitk_workspace_size(q1, k1, splits, None, True), dtype=torch.uint8, device=DEV)
    cu = [0, 1000, 4096, 8192]  # three packed sequences of 1000, 3096 and 4096 rows
    packed = [t.transpose(0, 1).reshape(H, B * N, D).contiguous() for t in (q1, k1, q2, k2)]
    pouts = tuple(torch.empty(H, B * N, device=DEV) for _ in range(3))
    pg = torch.full((H, B * N), 1e-3, device=DEV)
    pgrads = tuple(torch.empty(H, B * N, D, device=DEV) for _ in range(4))
    pws = torch.empty(bwd_varlen_workspace_size(packed[0], packed[1], cu, cu, None, True), dtype=torch.uint8,
                      device=DEV)

    def calls():
        streamkl_fwd(q1, k1, q2, k2, None, True, out=outs)
        streamkl_fwd_splitk(q1, k1, q2, k2, splits, None, True, workspace=wsk, out=outs)
        streamkl_bwd(q1, k1, q2, k2, *outs, g, None, True, workspace=ws, out=grads)
        streamkl_fwd_varlen(*packed, cu, cu, None, True, out=pouts)
        streamkl_bwd_varlen(*packed, cu, cu, *pouts, pg, None, True, workspace=pws, out=pgrads)
        torch.cuda.synchronize()

    calls()
    torch.cuda.reset_peak_memory_stats()
    held = torch.cuda.memory_allocated()
    free_before = torch.cuda.mem_get_info()[0]
    calls()
    assert torch.cuda.max_memory_allocated() == held
    assert torch.cuda.mem_get_info()[0] >= free_before


def test_autograd_function():
    q1, k1, q2, k2 = _rand(1, 2, 130, 260, 64, torch.float32, seed=9)
    ts = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
    kl = attention_kl(*ts, causal=True)
    (kl * 0.5).sum().backward()
    kl2, l1, l2 = streamkl_fwd(q1, k1, q2, k2, None, True)
    ref = streamkl_bwd(q1, k1, q2, k2, kl2, l1, l2, torch.full_like(kl2, 0.5), None, True)
    for t, r in zip(ts, ref):
        assert torch.equal(t.grad, r)


def test_errors_surface_as_exceptions():
    q1, k1, q2, k2 = _rand(1, 1, 16, 8, 128, torch.bfloat16, seed=10)
    with pytest.raises(StreamKLError):
        streamkl_fwd(q1, k1, q2, k2, None, True)  # causal with NQ > NK


# ------------------------------------------------------------ full-size workloads

def _full_size(name, rows_per_head=48, heads=None, bwd=True):
    w = synth.get(name)
    print(f"workload {name}", flush=True)
    q1, k1, q2, k2 = synth.make_inputs(w, device=DEV)
    heads = heads or [(0, 0), (w.B - 1, w.H - 1)]
    rows = sample_rows(w.NQ, rows_per_head, seed=w.cfg_id)
    if w.splits > 1:
        kl, l1, l2 = streamkl_fwd_splitk(q1, k1, q2, k2, w.splits, w.scale, w.causal)
    else:
        kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(kl).all() and torch.isfinite(l1).all() and torch.isfinite(l2).all()
    assert (kl >= -1e-5).all()
    assert_within(compare_forward(q1, k1, q2, k2, w.scale, w.causal, kl, l1, l2, heads, rows),
                  TOL[w.dtype], f"{name} fwd")
    if not bwd:
        return
    g = synth.upstream_grad(w, DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal)
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t).all()
    assert_within(compare_backward(q1, k1, q2, k2, w.scale, w.causal, g, grads, heads, rows, check_dk=False),
                  TOL[w.dtype], f"{name} dq")
    # Any-size invariant: key gradients of each head sum to zero.
    for dk in (grads[1], grads[3]):
        colsum = dk.double().sum(2).abs().max().item()
        assert colsum <= 1e-3 * dk.abs().max().item() * math.sqrt(w.NK), colsum
    del grads
    # Full dK check with g nonzero only on the sampled rows.
    gs = torch.zeros_like(g)
    gs[:, :, rows] = g[:, :, rows]
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, gs, w.scale, w.causal)
    torch.cuda.synchronize()
    assert_within(compare_backward(q1, k1, q2, k2, w.scale, w.causal, gs, grads, heads, rows, check_dk=True),
                  TOL[w.dtype], f"{name} dk (sampled g)")


def test_causal_4k_full_size():
    _full_size("causal_4k")


def test_noncausal_16k_full_size():
    _full_size("noncausal_16k")


def test_causal_64k_full_size():
    _full_size("causal_64k", rows_per_head=24)


def test_splitk_512k_forward_full_size():
    _full_size("splitk_512k", rows_per_head=24, bwd=False)


def test_splitk_bwd_128k_full_size():
    _full_size("splitk_bwd_128k", rows_per_head=24)


def test_causal_16k_d64_full_size():
    _full_size("causal_16k_d64")


def test_shortq_bwd_64k_full_size():
    # 2 query tiles per head: the query-gradient pass runs split over key chunks.
    _full_size("shortq_bwd_64k")


def test_shortq16_bwd_64k_full_size():
    # 16 queries per head: the fused single-visit backward.
    _full_size("shortq16_bwd_64k", rows_per_head=16)


def test_shortq128_bwd_64k_full_size():
    # 128 queries per head: the fused backward with four query blocks per workgroup.
    _full_size("shortq128_bwd_64k", rows_per_head=32)


FUSED = [
    # B, H, NQ, NK, D, causal: at most 128 queries per unit take the fused
    # single-visit backward (one block of 32 queries per workgroup up to 32,
    # four above); ragged query and key blocks, one and several key chunks.
    (1, 2, 1, 37, 128, False),
    (1, 2, 5, 1000, 128, True),
    (2, 1, 16, 5000, 128, False),
    (1, 3, 32, 4130, 64, True),
    (1, 1, 32, 32, 128, True),
    (2, 2, 17, 777, 64, False),
    (1, 2, 33, 900, 128, True),
    (2, 1, 100, 3000, 128, False),
    (1, 2, 128, 2100, 64, True),
    (1, 1, 128, 128, 128, False),
]


@pytest.mark.parametrize("B,H,NQ,NK,D,causal", FUSED)
def test_fused_short_query_backward(B, H, NQ, NK, D, causal):
    # The combined call runs the fused kernel; the step-wise calls run the
    # split passes.  Both against the oracle, element by element, with signed
    # g, and each distribution's gradients alone equal to the combined call's.
    from attention_kl_divergence_online_amd import streamkl_bwd_dk, streamkl_bwd_dq, streamkl_bwd_prepare
    print(f"fused B={B} H={H} NQ={NQ} NK={NK} D={D} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, torch.bfloat16, seed=NQ * 31 + NK + D + causal, noise=0.2)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    g = (torch.rand((B, H, NQ), generator=torch.Generator().manual_seed(NK)) - 0.3).to(DEV)
    fused = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    ws = streamkl_bwd_prepare(q1, k1, q2, k2, g, scale, causal)
    dk1, dk2 = streamkl_bwd_dk(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, workspace=ws)
    dq1, dq2 = streamkl_bwd_dq(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, workspace=ws)
    t_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, student=False)
    s_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, teacher=False)
    torch.cuda.synchronize()
    heads = _heads(B, H)
    case = f"B{B} H{H} NQ{NQ} NK{NK} D{D} causal={causal}"
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, fused, heads), TOL["bf16"], f"fused {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, (dq1, dk1, dq2, dk2), heads), TOL["bf16"],
                  f"split {case}")
    for a, b in ((t_only[0], fused[0]), (t_only[1], fused[1]), (s_only[2], fused[2]), (s_only[3], fused[3])):
        assert torch.equal(a, b)


def test_causal_4k_fp32_full_size():
    _full_size("causal_4k_fp32")


def test_decode_128k_full_size():
    # Every one of the 16 rows of two heads, and the backward of the decode shape.
    _full_size("decode_128k", rows_per_head=16)


def _sweep_cases(n=24, seed=2026):
    # Seeded draws of small problems: ragged lengths on both sides, NQ <= NK
    # when causal, both head sizes, a few heads and batches.
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        causal = bool(rng.integers(0, 2))
        nk = int(rng.integers(1, 900))
        nq = int(rng.integers(1, nk + 1)) if causal else int(rng.integers(1, 900))
        cases.append((int(rng.integers(1, 3)), int(rng.integers(1, 4)), nq, nk, int(rng.choice([64, 128])), causal))
    return cases


@pytest.mark.parametrize("B,H,NQ,NK,D,causal", _sweep_cases())
def test_seeded_shape_sweep_bf16(B, H, NQ, NK, D, causal):
    print(f"sweep B={B} H={H} NQ={NQ} NK={NK} D={D} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand(B, H, NQ, NK, D, torch.bfloat16, seed=NQ * 13 + NK * 7 + D + causal)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    gen = torch.Generator(device="cpu").manual_seed(NQ + NK)
    g = torch.rand(B, H, NQ, generator=gen).mul_(2).sub_(0.5).to(DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    heads = _heads(B, H)
    case = f"sweep B{B} H{H} NQ{NQ} NK{NK} D{D} causal={causal}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"], f"fwd {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, grads, heads), TOL["bf16"], f"bwd {case}")


def test_mfma_rate_probe_runs():
    # The measurement helper: about 1.4 GFLOP of register-only products; the
    # rate must be a plausible fraction of the 2.5 PFLOP/s bf16 peak.
    from attention_kl_divergence_online_amd import streamkl_probe_mfma_bf16
    wg, iters = 256, 2000
    sink = torch.zeros(4 * wg, device=DEV)
    streamkl_probe_mfma_bf16(iters, wg, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    streamkl_probe_mfma_bf16(iters, wg, sink)
    e1.record()
    torch.cuda.synchronize()
    tflops = wg * 4 * iters * 4 * 32768 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"probe {tflops:.0f} TFLOP/s", flush=True)
    assert torch.isfinite(sink).all()
    assert 200.0 < tflops < 2600.0
