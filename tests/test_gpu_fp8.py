"""GPU parity of the fp8 (e4m3) forward and backward against the fp64 oracle.

The inputs are fp8 values (seeded normals rounded to e4m3), and the oracle is
given exactly those values in fp64, so the only differences are the kernels'
fp32 accumulation, exponentials and the backward's 16-bit dS: the bf16 path's
2e-3 bound applies.  Shapes cover the four-wave and twelve-wave fp8 forward
shapes, both backward passes (with the query pass split over key chunks for
few query tiles), both head dimensions, ragged tails in N_Q and N_K, the
causal diagonal, single-distribution passes, the fused single-visit backward
of at most 128 queries against the split passes, split-K chunks, a packed
variable-length batch and the causal 64K workload's full size.
"""
import math

import numpy as np
import pytest
import torch

import synth
from attention_kl_divergence_online_amd import (streamkl_bwd, streamkl_bwd_varlen, streamkl_fwd, streamkl_fwd_splitk,
                                                streamkl_fwd_varlen)
from parity_util import TOL, assert_within, compare_backward, compare_forward, sample_rows

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not hasattr(torch, "float8_e4m3fn"), reason="torch without float8 types")]

DEV = "cuda"


def _rand_fp8(shape_q, shape_k, seed, noise=0.3):
    g = torch.Generator(device="cpu").manual_seed(seed)
    q1 = torch.randn(*shape_q, generator=g)
    k1 = torch.randn(*shape_k, generator=g)
    q2 = q1 + noise * torch.randn(*shape_q, generator=g)
    k2 = k1 + noise * torch.randn(*shape_k, generator=g)
    return [synth.to_fp8(t).to(DEV).contiguous() for t in (q1, k1, q2, k2)]


CASES = [
    # B, H, NQ, NK, D, causal
    (1, 2, 300, 517, 128, False),
    (1, 2, 300, 517, 128, True),
    (2, 1, 700, 700, 128, True),     # four-wave causal shape
    (1, 3, 129, 1000, 64, False),
    (1, 2, 257, 333, 64, True),
    (1, 1, 1, 37, 128, False),
    (1, 1, 5, 5, 128, True),
    (2, 1, 16, 77, 64, True),        # at most 32 queries: the one-wave decode shape (32-key tiles)
    (2, 2, 32, 1500, 128, True),     # the decode shape at its 32-query limit
    (1, 1, 33, 900, 128, False),     # one query past it: the twelve-wave shape
    (1, 1, 4160, 4160, 128, True),   # twelve-wave causal shape, 128-key tiles
    (1, 2, 1000, 2500, 128, False),  # twelve-wave non-causal shape, ragged last query tile
]


def _grad(B, H, NQ, seed):
    # Upstream gradients of mixed sign (the key pass's signed-dS variant).
    g = torch.Generator(device="cpu").manual_seed(seed)
    return (torch.randn(B, H, NQ, generator=g) / (B * H * NQ)).to(DEV)


@pytest.mark.parametrize("B,H,NQ,NK,D,causal", CASES)
def test_fp8_forward_backward_all_rows(B, H, NQ, NK, D, causal):
    print(f"fp8 B={B} H={H} NQ={NQ} NK={NK} D={D} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand_fp8((B, H, NQ, D), (B, H, NK, D), seed=NQ * 5 + NK + D + causal)
    scale = D ** -0.5
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    assert torch.isfinite(kl).all() and torch.isfinite(l1).all() and torch.isfinite(l2).all()
    what = f"NQ={NQ} NK={NK} D={D} causal={causal}"
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"], f"fp8 fwd {what}")
    g = _grad(B, H, NQ, seed=NQ + NK)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t).all()
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, grads, heads), TOL["bf16"], f"fp8 bwd {what}")


FUSED = [
    # B, H, NQ, NK, D, causal: at most 128 queries per unit take the fused
    # single-visit backward (one or four 32-query blocks per workgroup).
    (1, 2, 5, 1000, 128, True),
    (2, 1, 16, 5000, 128, False),
    (1, 3, 32, 4130, 64, True),
    (2, 1, 100, 3000, 128, False),
    (1, 2, 128, 2100, 64, True),
]


@pytest.mark.parametrize("B,H,NQ,NK,D,causal", FUSED)
def test_fp8_fused_short_query_backward(B, H, NQ, NK, D, causal):
    # The combined call runs the fused kernel, the step-wise calls the split
    # passes; both against the oracle with signed g, and each distribution's
    # gradients alone equal to the combined call's.
    from attention_kl_divergence_online_amd import streamkl_bwd_dk, streamkl_bwd_dq, streamkl_bwd_prepare
    print(f"fp8 fused B={B} H={H} NQ={NQ} NK={NK} D={D} causal={causal}", flush=True)
    q1, k1, q2, k2 = _rand_fp8((B, H, NQ, D), (B, H, NK, D), seed=NQ * 31 + NK + D + causal, noise=0.2)
    scale = D ** -0.5
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    g = _grad(B, H, NQ, seed=NK)
    fused = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    ws = streamkl_bwd_prepare(q1, k1, q2, k2, g, scale, causal)
    dk1, dk2 = streamkl_bwd_dk(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, workspace=ws)
    dq1, dq2 = streamkl_bwd_dq(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, workspace=ws)
    t_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, student=False)
    s_only = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, teacher=False)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(H)]
    case = f"B{B} H{H} NQ{NQ} NK{NK} D{D} causal={causal}"
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, fused, heads), TOL["bf16"], f"fp8 fused {case}")
    assert_within(compare_backward(q1, k1, q2, k2, scale, causal, g, (dq1, dk1, dq2, dk2), heads), TOL["bf16"],
                  f"fp8 split {case}")
    for a, b in ((t_only[0], fused[0]), (t_only[1], fused[1]), (s_only[2], fused[2]), (s_only[3], fused[3])):
        assert torch.equal(a, b)


@pytest.mark.parametrize("teacher,student", [(True, False), (False, True)])
def test_fp8_single_distribution_passes(teacher, student):
    B, H, NQ, NK, D, causal = 1, 2, 300, 517, 128, True
    print(f"fp8 teacher={teacher} student={student}", flush=True)
    q1, k1, q2, k2 = _rand_fp8((B, H, NQ, D), (B, H, NK, D), seed=99)
    scale = D ** -0.5
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
    g = _grad(B, H, NQ, seed=5)
    both = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal)
    one = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, scale, causal, teacher=teacher, student=student)
    torch.cuda.synchronize()
    # The single-distribution passes accumulate in the same order as the full one.
    for a, b in zip(both, one):
        if b is not None:
            assert torch.equal(a, b)


@pytest.mark.parametrize("causal,NQ", [(False, 200), (True, 200), (True, 16)])
def test_fp8_splitk_matches_oracle(causal, NQ):
    B, H, NK, D = 1, 2, 3000, 128
    print(f"fp8 split-K causal={causal} NQ={NQ}", flush=True)
    q1, k1, q2, k2 = _rand_fp8((B, H, NQ, D), (B, H, NK, D), seed=77 + causal)
    scale = D ** -0.5
    kl, l1, l2 = streamkl_fwd_splitk(q1, k1, q2, k2, 5, scale, causal)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 1)]
    assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"],
                  f"fp8 split fwd causal={causal} NQ={NQ}")


def test_fp8_varlen_matches_per_sequence_oracle():
    lens_q, lens_k, H, D, causal = [1, 130, 0, 300, 64], [5, 130, 9, 517, 64], 2, 128, True
    print("fp8 varlen", flush=True)
    TQ, TK = sum(lens_q), sum(lens_k)
    q1, k1, q2, k2 = _rand_fp8((H, TQ, D), (H, TK, D), seed=4242)
    cu_q, cu_k = [0] + np.cumsum(lens_q).tolist(), [0] + np.cumsum(lens_k).tolist()
    scale = D ** -0.5
    kl, l1, l2 = streamkl_fwd_varlen(q1, k1, q2, k2, cu_q, cu_k, scale, causal)
    g = _grad(1, H, TQ, seed=11)[0]
    grads = streamkl_bwd_varlen(q1, k1, q2, k2, cu_q, cu_k, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(H)]
    for b in range(len(lens_q)):
        sq, sk = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
        if lens_q[b] == 0:
            for dk in (grads[1], grads[3]):
                assert not dk[:, sk].any()  # no queries: zero key gradients
            continue
        seq = [t[:, s].unsqueeze(0) for t, s in ((q1, sq), (k1, sk), (q2, sq), (k2, sk))]
        outs = [t[:, sq].unsqueeze(0) for t in (kl, l1, l2)]
        assert_within(compare_forward(*seq, scale, causal, *outs, heads), TOL["bf16"], f"fp8 varlen seq {b}")
        sg = [t[:, s].unsqueeze(0) for t, s in zip(grads, (sq, sk, sq, sk))]
        assert_within(compare_backward(*seq, scale, causal, g[:, sq].unsqueeze(0), sg, heads), TOL["bf16"],
                      f"fp8 varlen bwd seq {b}")


def test_fp8_causal_64k_sampled_rows():
    # The causal 64K workload's shape (32 heads) with its inputs rounded to
    # e4m3, in the launches the bench times: sampled rows of two heads for the
    # forward and dQ, the whole dK with g nonzero only on those rows (dK is
    # linear in g), and the any-size invariant sum_j dK[j] = 0.
    w = synth.get("causal_64k")
    print("fp8 causal 64K", flush=True)
    q1, k1, q2, k2 = (synth.to_fp8(t) for t in synth.make_inputs(w, DEV))
    kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, w.scale, w.causal)
    torch.cuda.synchronize()
    rows = sample_rows(w.NQ, 24, seed=5)
    heads = [(0, 0), (0, w.H - 1)]
    assert_within(compare_forward(q1, k1, q2, k2, w.scale, w.causal, kl, l1, l2, heads, rows=rows), TOL["bf16"],
                  "fp8 causal_64k fwd (sampled rows)")
    g = synth.upstream_grad(w, DEV)
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, g, w.scale, w.causal)
    torch.cuda.synchronize()
    assert_within(compare_backward(q1, k1, q2, k2, w.scale, w.causal, g, grads, heads, rows, check_dk=False),
                  TOL["bf16"], "fp8 causal_64k dq")
    for dk in (grads[1], grads[3]):
        colsum = dk.double().sum(2).abs().max().item()
        assert colsum <= 1e-3 * dk.abs().max().item() * math.sqrt(w.NK), colsum
    del grads
    gs = torch.zeros_like(g)
    gs[:, :, rows] = g[:, :, rows]
    grads = streamkl_bwd(q1, k1, q2, k2, kl, l1, l2, gs, w.scale, w.causal)
    torch.cuda.synchronize()
    assert_within(compare_backward(q1, k1, q2, k2, w.scale, w.causal, gs, grads, heads, rows, check_dk=True),
                  TOL["bf16"], "fp8 causal_64k dk (sampled g)")


@pytest.mark.parametrize("offset", [1000.0, 1400.0])
def test_fp8_teacher_maxima_far_above_the_students(offset):
    # As the bf16 case in test_gpu_parity.py: the teacher's keys share a
    # component along its queries' direction, so its held maxima sit about
    # 0.127 * offset log2 units above the student's, near the forward's
    # 160-unit span for one shared exponent offset (1000) and past it (1400),
    # here with the fp8 instruction's inexact sums in x1 - x2.
    B, H, NQ, NK, D = 1, 2, 700, 1500, 128
    print(f"fp8 far-apart maxima offset={offset}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(int(offset) + 3)
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    q1 = (offset / 10.0) * u + 0.7 * torch.randn(B, H, NQ, D, generator=g)
    k1 = 10.0 * u + 0.3 * torch.randn(B, H, NK, D, generator=g)
    q2 = torch.randn(B, H, NQ, D, generator=g)
    k2 = torch.randn(B, H, NK, D, generator=g)
    q1, k1, q2, k2 = (synth.to_fp8(t).to(DEV).contiguous() for t in (q1, k1, q2, k2))
    scale = D ** -0.5
    heads = [(b, h) for b in range(B) for h in range(H)]
    for causal in (False, True):
        kl, l1, l2 = streamkl_fwd(q1, k1, q2, k2, scale, causal)
        kls, l1s, l2s = streamkl_fwd_splitk(q1, k1, q2, k2, 3, scale, causal)
        torch.cuda.synchronize()
        what = f"offset={offset} causal={causal}"
        assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kl, l1, l2, heads), TOL["bf16"],
                      f"fp8 fwd far-apart {what}")
        assert_within(compare_forward(q1, k1, q2, k2, scale, causal, kls, l1s, l2s, heads), TOL["bf16"],
                      f"fp8 split fwd far-apart {what}")
