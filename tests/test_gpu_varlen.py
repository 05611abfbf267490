"""GPU parity of packed variable-length batches (streamkl_fwd_varlen,
streamkl_bwd_varlen).

Every sequence of a packed batch is an independent problem, so the reference
is the fp64 oracle applied to each sequence's slice of the packed tensors,
element by element at small sizes.  With equal lengths a packed batch is a
permutation of a dense [B, H, N, D] problem, and the results must equal the
dense entry points' bit for bit.  The 16-sequence mixed-length batch the
benchmark times is checked on sampled rows plus the per-sequence invariant
sum_j dK[j] = 0.
"""
import math

import numpy as np
import pytest
import torch

import synth
from attention_kl_divergence_online_amd import (attention_kl_varlen, streamkl_bwd, streamkl_bwd_varlen,
                                                streamkl_fwd, streamkl_fwd_varlen)
from parity_util import TOL, assert_within, compare_backward, compare_forward, sample_rows

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _cu(lens):
    return [0] + np.cumsum(lens).tolist()


def _packed(lens_q, lens_k, H, D, dtype, seed, noise=0.3):
    gen = torch.Generator(device="cpu").manual_seed(seed)
    TQ, TK = sum(lens_q), sum(lens_k)
    q1 = torch.randn(H, TQ, D, generator=gen)
    k1 = torch.randn(H, TK, D, generator=gen)
    q2 = q1 + noise * torch.randn(H, TQ, D, generator=gen)
    k2 = k1 + noise * torch.randn(H, TK, D, generator=gen)
    return [t.to(dtype).to(DEV).contiguous() for t in (q1, k1, q2, k2)]


def _seq(t, c0, c1):
    """Sequence rows [c0, c1) of a packed [H, T, ...] tensor as a [1, H, c1-c0, ...] view."""
    return t[:, c0:c1].unsqueeze(0)


CASES = [
    # lens_q, lens_k, D, causal, dtype.  Runs of equal lengths (40 x 3), a sequence with
    # no queries, one with neither, ragged tails around the 64/128/256-row tiles.
    ([1, 17, 64, 0, 130, 40, 40, 40, 0, 300], [5, 17, 200, 9, 130, 40, 40, 40, 0, 517], 128, False, "bf16"),
    ([1, 17, 64, 0, 130, 40, 40, 40, 0, 300], [5, 17, 200, 9, 130, 40, 40, 40, 0, 517], 128, True, "bf16"),
    ([257, 3, 3, 129], [257, 70, 70, 400], 64, True, "bf16"),
    ([33, 0, 190, 190, 7], [100, 12, 190, 190, 7], 128, True, "fp32"),
    ([65, 5], [300, 64], 64, False, "fp32"),
    # A causal batch with a sequence past 8192 rows: the forward's shared
    # launch takes the eight-wave, 128-key-tile shape for every sequence.
    ([9000, 300], [9000, 300], 128, True, "bf16"),
]


@pytest.mark.parametrize("lens_q,lens_k,D,causal,dt", CASES)
def test_varlen_matches_oracle_per_sequence(lens_q, lens_k, D, causal, dt):
    H = 2
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    print(f"varlen lens_q={lens_q} lens_k={lens_k} D={D} causal={causal} {dt}", flush=True)
    q1, k1, q2, k2 = _packed(lens_q, lens_k, H, D, dtype, seed=sum(lens_q) + 7 * D + causal)
    cq, ck = _cu(lens_q), _cu(lens_k)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd_varlen(q1, k1, q2, k2, cq, ck, scale, causal)
    # Signed, uneven upstream gradient: exercises the per-sequence dS scaling and sign paths.
    gen = torch.Generator(device="cpu").manual_seed(11)
    g = (torch.randn(H, cq[-1], generator=gen) * 1e-3).to(DEV).contiguous()
    grads = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(H)]
    for b in range(len(lens_q)):
        q0, q1e, k0, k1e = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if q1e == q0:
            # No query rows: the sequence's key gradients are zero.
            for dk in (grads[1], grads[3]):
                assert torch.count_nonzero(dk[:, k0:k1e]).item() == 0
            continue
        S = lambda t, a, e: _seq(t, a, e)
        sq = [S(q1, q0, q1e), S(k1, k0, k1e), S(q2, q0, q1e), S(k2, k0, k1e)]
        errs = compare_forward(*sq, scale, causal, S(kl, q0, q1e), S(l1, q0, q1e), S(l2, q0, q1e), heads)
        assert_within(errs, TOL[dt], f"varlen fwd seq {b} ({q1e - q0}x{k1e - k0})")
        sg = [S(grads[0], q0, q1e), S(grads[1], k0, k1e), S(grads[2], q0, q1e), S(grads[3], k0, k1e)]
        errs = compare_backward(*sq, scale, causal, S(g, q0, q1e), sg, heads)
        assert_within(errs, TOL[dt], f"varlen bwd seq {b} ({q1e - q0}x{k1e - k0})")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_equal_dense(causal):
    # Packed [H, B*N, D] with B equal sequences is the dense [B, H, N, D] problem with
    # another layout: same kernels, same per-(sequence, head) arithmetic, same bits.
    B, H, N, D = 3, 2, 200, 128
    print(f"varlen vs dense B={B} H={H} N={N} causal={causal}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(5)
    dense = [torch.randn(B, H, N, D, generator=gen).to(torch.bfloat16).to(DEV) for _ in range(4)]
    g = (torch.rand(B, H, N, generator=gen) - 0.3).to(DEV)
    pack = lambda t: t.transpose(0, 1).reshape(H, B * N, *t.shape[3:]).contiguous()
    unpack = lambda t: t.reshape(H, B, N, *t.shape[2:]).transpose(0, 1)
    scale = 0.1
    out_d = streamkl_fwd(*dense, scale, causal)
    grads_d = streamkl_bwd(*dense, *out_d, g, scale, causal)
    cu = [0, N, 2 * N, 3 * N]
    packed = [pack(t) for t in dense]
    out_v = streamkl_fwd_varlen(*packed, cu, cu, scale, causal)
    grads_v = streamkl_bwd_varlen(*packed, cu, cu, *out_v, pack(g), scale, causal)
    torch.cuda.synchronize()
    for a, b in zip(out_d, out_v):
        assert torch.equal(a, unpack(b))
    for a, b in zip(grads_d, grads_v):
        assert torch.equal(a, unpack(b))


def test_varlen_segmented_equal_lengths_equal_dense():
    # 3 x 16 x 6 = 288 query tiles fill the GPU, so the packed batch takes the
    # segmented passes (one launch over all runs); with equal lengths it is the
    # dense problem with another layout and must give the same bits.
    B, H, N, D = 3, 16, 700, 64
    print(f"segmented varlen vs dense B={B} H={H} N={N}", flush=True)
    gen = torch.Generator(device="cpu").manual_seed(8)
    dense = [torch.randn(B, H, N, D, generator=gen).to(torch.bfloat16).to(DEV) for _ in range(4)]
    g = (torch.rand(B, H, N, generator=gen) - 0.3).to(DEV)
    pack = lambda t: t.transpose(0, 1).reshape(H, B * N, *t.shape[3:]).contiguous()
    unpack = lambda t: t.reshape(H, B, N, *t.shape[2:]).transpose(0, 1)
    out_d = streamkl_fwd(*dense, None, True)
    grads_d = streamkl_bwd(*dense, *out_d, g, None, True)
    cu = [0, N, 2 * N, 3 * N]
    packed = [pack(t) for t in dense]
    out_v = streamkl_fwd_varlen(*packed, cu, cu, None, True)
    grads_v = streamkl_bwd_varlen(*packed, cu, cu, *out_v, pack(g), None, True)
    torch.cuda.synchronize()
    for a, b in zip(out_d, out_v):
        assert torch.equal(a, unpack(b))
    for a, b in zip(grads_d, grads_v):
        assert torch.equal(a, unpack(b))


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_varlen_many_runs(dt):
    # 43 runs: more than one segmented launch holds (32 segments), runs of the
    # main forward shape mixed with decode-shaped ones (at most 32 queries), a
    # query-less sequence and a run of two equal sequences; 8 heads give 376
    # query tiles, so every run joins the segmented backward passes.
    # (fp32 has no decode shape; its shortest sequence has 6 queries, since the
    # error measure of a one-row slice is that row's relative KL error, which
    # fp32 cancellation in a KL near 0.02 takes past 1e-5 in any launch.)
    H, D, causal = 8, 64, True
    lens_q = [33 + 3 * i for i in range(36)] + [1 if dt == "bf16" else 6, 16, 32, 0, 5, 20, 90, 90]
    lens_k = [n + (i % 5) * 7 for i, n in enumerate(lens_q)]
    lens_k[39] = 11
    lens_k[43] = lens_k[42]
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    print(f"varlen {len(lens_q)} sequences {dt}", flush=True)
    q1, k1, q2, k2 = _packed(lens_q, lens_k, H, D, dtype, seed=21)
    cq, ck = _cu(lens_q), _cu(lens_k)
    scale = 1.0 / math.sqrt(D)
    kl, l1, l2 = streamkl_fwd_varlen(q1, k1, q2, k2, cq, ck, scale, causal)
    gen = torch.Generator(device="cpu").manual_seed(12)
    g = (torch.randn(H, cq[-1], generator=gen) * 1e-3).to(DEV).contiguous()
    grads = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, kl, l1, l2, g, scale, causal)
    torch.cuda.synchronize()
    heads = [(0, h) for h in range(H)]
    for b in range(len(lens_q)):
        q0, qe, k0, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        if qe == q0:
            for dk in (grads[1], grads[3]):
                assert torch.count_nonzero(dk[:, k0:ke]).item() == 0
            continue
        S = _seq
        sq = [S(q1, q0, qe), S(k1, k0, ke), S(q2, q0, qe), S(k2, k0, ke)]
        errs = compare_forward(*sq, scale, causal, S(kl, q0, qe), S(l1, q0, qe), S(l2, q0, qe), heads)
        assert_within(errs, TOL[dt], f"varlen many-run fwd seq {b} ({qe - q0}x{ke - k0}) {dt}")
        sg = [S(grads[0], q0, qe), S(grads[1], k0, ke), S(grads[2], q0, qe), S(grads[3], k0, ke)]
        errs = compare_backward(*sq, scale, causal, S(g, q0, qe), sg, heads)
        assert_within(errs, TOL[dt], f"varlen many-run bwd seq {b} ({qe - q0}x{ke - k0}) {dt}")
        if b in (0, 35, 36, 38, 42):
            # The same sequence as a dense problem of its own, through the
            # step-wise entry points (always the split passes, which the
            # packed batch runs too; the combined call would take the fused
            # pass for sequences of at most 32 queries): the same bits forward
            # and for dK.  The dense dQ pass of so few query tiles splits its
            # keys and sums the chunks' partials afterwards, so dQ differs by
            # fp32 summation order only.
            from attention_kl_divergence_online_amd import streamkl_bwd_dk, streamkl_bwd_dq, streamkl_bwd_prepare
            dq = [t.contiguous() for t in sq]
            out_d = streamkl_fwd(*dq, scale, causal)
            gd = S(g, q0, qe).contiguous()
            wsd = streamkl_bwd_prepare(*dq, gd, scale, causal)
            dk1d, dk2d = streamkl_bwd_dk(*dq, *out_d, gd, scale, causal, workspace=wsd)
            dq1d, dq2d = streamkl_bwd_dq(*dq, *out_d, gd, scale, causal, workspace=wsd)
            grads_d = (dq1d, dk1d, dq2d, dk2d)
            torch.cuda.synchronize()
            for a, c in zip(out_d, (S(kl, q0, qe), S(l1, q0, qe), S(l2, q0, qe))):
                assert torch.equal(a, c), b
            for i in (1, 3):
                assert torch.equal(grads_d[i], sg[i]), b
            for i in (0, 2):
                d = (grads_d[i] - sg[i]).abs().max().item() / sg[i].abs().max().item()
                assert d <= 1e-5, (b, i, d)


def test_varlen_teacher_or_student_only():
    lens_q, lens_k = [130, 0, 77], [200, 9, 77]
    H, D = 2, 128
    print("varlen single-distribution gradients", flush=True)
    q1, k1, q2, k2 = _packed(lens_q, lens_k, H, D, torch.bfloat16, seed=3)
    cq, ck = _cu(lens_q), _cu(lens_k)
    out = streamkl_fwd_varlen(q1, k1, q2, k2, cq, ck, None, True)
    g = torch.full((H, cq[-1]), 1e-2, device=DEV)
    both = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, *out, g, None, True)
    teacher = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, *out, g, None, True, student=False)
    student = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, *out, g, None, True, teacher=False)
    torch.cuda.synchronize()
    assert teacher[2] is None and student[0] is None
    for i in (0, 1):
        assert torch.equal(teacher[i], both[i])
    for i in (2, 3):
        assert torch.equal(student[i], both[i])


def test_varlen_autograd_matches_direct_calls():
    lens_q, lens_k = [70, 0, 129], [70, 5, 300]
    H, D = 2, 64
    print("varlen autograd", flush=True)
    q1, k1, q2, k2 = _packed(lens_q, lens_k, H, D, torch.float32, seed=9)
    cq, ck = _cu(lens_q), _cu(lens_k)
    leaves = [t.clone().requires_grad_(True) for t in (q1, k1, q2, k2)]
    kl = attention_kl_varlen(*leaves, cq, ck, None, True)
    gen = torch.Generator(device="cpu").manual_seed(4)
    w = torch.randn(kl.shape, generator=gen).to(DEV)
    (kl * w).sum().backward()
    out = streamkl_fwd_varlen(q1, k1, q2, k2, cq, ck, None, True)
    grads = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, *out, w.contiguous(), None, True)
    torch.cuda.synchronize()
    assert torch.equal(kl.detach(), out[0])
    for leaf, gr in zip(leaves, grads):
        assert torch.equal(leaf.grad, gr)


def test_varlen_mix_full_size():
    # The benchmark's packed batch: 16 causal sequences of 1K-7K tokens, 32 heads, D 128.
    pb = synth.PACKED["varlen_mix"]
    print(f"packed batch {pb.name}: {len(pb.lens_q)} sequences, {pb.cu_q[-1]} rows", flush=True)
    q1, k1, q2, k2 = synth.make_packed(pb, DEV)
    cq, ck = pb.cu_q, pb.cu_k
    kl, l1, l2 = streamkl_fwd_varlen(q1, k1, q2, k2, cq, ck, pb.scale, pb.causal)
    g = synth.packed_grad(pb, DEV)
    grads = streamkl_bwd_varlen(q1, k1, q2, k2, cq, ck, kl, l1, l2, g, pb.scale, pb.causal)
    torch.cuda.synchronize()
    for t in (kl, l1, l2) + tuple(grads):
        assert torch.isfinite(t).all()
    assert (kl >= -1e-5).all()
    heads = [(0, 0), (0, pb.H - 1)]
    longest = max(range(len(pb.lens_q)), key=lambda b: pb.lens_q[b])
    for b in sorted({0, longest, len(pb.lens_q) - 1}):
        q0, qe, k0, ke = cq[b], cq[b + 1], ck[b], ck[b + 1]
        rows = sample_rows(qe - q0, 24, seed=b)
        S = _seq
        sq = [S(q1, q0, qe), S(k1, k0, ke), S(q2, q0, qe), S(k2, k0, ke)]
        errs = compare_forward(*sq, pb.scale, pb.causal, S(kl, q0, qe), S(l1, q0, qe), S(l2, q0, qe), heads,
                               rows)
        assert_within(errs, TOL[pb.dtype], f"{pb.name} fwd seq {b}")
        sg = [S(grads[0], q0, qe), S(grads[1], k0, ke), S(grads[2], q0, qe), S(grads[3], k0, ke)]
        errs = compare_backward(*sq, pb.scale, pb.causal, S(g, q0, qe), sg, heads, rows, check_dk=False)
        assert_within(errs, TOL[pb.dtype], f"{pb.name} dq seq {b}")
    # Any-size invariant per (sequence, head): key gradients sum to zero over the keys.
    for dk in (grads[1], grads[3]):
        for b in range(len(pb.lens_k)):
            part = dk[:, ck[b]:ck[b + 1]].double()
            colsum = part.sum(1).abs().max().item()
            assert colsum <= 1e-3 * part.abs().max().item() * math.sqrt(pb.lens_k[b]), (b, colsum)
