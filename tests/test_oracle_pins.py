"""Pins of the fp64 oracle to things other than itself.

The oracle (oracle/streamkl_oracle.c) computes per-row KL(P1||P2), LSE1, LSE2
and the gradients of sum_i g_i KL_i.  Each test below checks it against an
independent route: a high-precision brute force through probabilities
(mpmath), library routines (torch.kl_div / logsumexp, scipy entropy, torch
autograd), closed forms, invariants, finite differences, and the pages' own
online recurrence (gist.science "Formulacion Online").  Any of a dropped term,
a sign error, a transposed operand, an off-by-one causal mask or a wrong scale
fails at least one of them (tests/test_oracle_mutants.py plants such mistakes in a
copy of the oracle and checks that they are caught).
"""
import math

import mpmath
import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
from oracle import online, reference_mp

# (NQ, NK, D, causal): square, rectangular, bottom-right causal with NQ < NK.
SHAPES = [(5, 7, 4, False), (5, 7, 4, True), (6, 6, 3, True), (1, 9, 2, False), (8, 3, 5, False),
          (4, 4, 8, False), (3, 8, 2, True)]


def _inputs(nq, nk, d, seed, std=1.0, noise=0.5):
    rng = np.random.default_rng(seed)
    q1 = rng.standard_normal((nq, d)) * std
    k1 = rng.standard_normal((nk, d)) * std
    q2 = q1 + noise * rng.standard_normal((nq, d))
    k2 = k1 + noise * rng.standard_normal((nk, d))
    return q1, k1, q2, k2


def _visible(nq, nk, causal):
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return np.ones((nq, nk), bool) if not causal else (j <= i + (nk - nq))


@pytest.mark.parametrize("nq,nk,d,causal", SHAPES)
def test_forward_matches_mpmath_brute_force(oracle_lib, nq, nk, d, causal):
    q1, k1, q2, k2 = _inputs(nq, nk, d, seed=nq * 100 + nk)
    scale = 0.7
    kl, l1, l2 = oracle.fwd(q1, k1, q2, k2, scale, causal)
    mkl, ml1, ml2 = reference_mp.kl_rows(q1.tolist(), k1.tolist(), q2.tolist(), k2.tolist(), scale, causal)
    for a, b in ((kl, mkl), (l1, ml1), (l2, ml2)):
        b = np.array([float(x) for x in b])
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("nq,nk,d,causal", SHAPES)
def test_forward_matches_torch_kl_div(oracle_lib, nq, nk, d, causal):
    q1, k1, q2, k2 = _inputs(nq, nk, d, seed=7 + nq + nk)
    scale = 1.0 / math.sqrt(d)
    kl, l1, l2 = oracle.fwd(q1, k1, q2, k2, scale, causal)
    vis = _visible(nq, nk, causal)
    t = lambda a: torch.from_numpy(a)
    s1 = scale * t(q1) @ t(k1).T
    s2 = scale * t(q2) @ t(k2).T
    for i in range(nq):
        m = t(vis[i])
        ls1 = torch.log_softmax(s1[i][m], -1)
        ls2 = torch.log_softmax(s2[i][m], -1)
        ref = torch.nn.functional.kl_div(ls2, ls1, log_target=True, reduction="sum").item()
        assert kl[i] == pytest.approx(ref, rel=1e-12, abs=1e-14)
        assert l1[i] == pytest.approx(torch.logsumexp(s1[i][m], -1).item(), rel=1e-13)
        assert l2[i] == pytest.approx(torch.logsumexp(s2[i][m], -1).item(), rel=1e-13)


def test_zero_queries_give_uniform_rows(oracle_lib):
    # Q1 = Q2 = 0: both rows uniform over the n_i visible keys -> KL = 0, LSE = ln n_i.
    nq, nk, d = 6, 9, 4
    rng = np.random.default_rng(1)
    for causal in (False, True):
        z = np.zeros((nq, d))
        kl, l1, l2 = oracle.fwd(z, rng.standard_normal((nk, d)), z, rng.standard_normal((nk, d)), 0.5, causal)
        n = _visible(nq, nk, causal).sum(1)
        np.testing.assert_allclose(kl, 0.0, atol=1e-15)
        np.testing.assert_allclose(l1, np.log(n), rtol=1e-15)
        np.testing.assert_allclose(l2, np.log(n), rtol=1e-15)


def test_uniform_student_gives_log_n_minus_entropy(oracle_lib):
    # Q2 = 0: P2 uniform, KL = ln n_i - H(P1) with H from scipy.
    nq, nk, d = 5, 11, 3
    q1, k1, _, k2 = _inputs(nq, nk, d, seed=3)
    scale = 0.9
    for causal in (False, True):
        kl, _, _ = oracle.fwd(q1, k1, np.zeros_like(q1), k2, scale, causal)
        vis = _visible(nq, nk, causal)
        for i in range(nq):
            s = scale * (k1[vis[i]] @ q1[i])
            p = scipy.special.softmax(s)
            assert kl[i] == pytest.approx(math.log(vis[i].sum()) - scipy.stats.entropy(p), rel=1e-11, abs=1e-14)


def test_uniform_teacher(oracle_lib):
    # Q1 = 0: P1 uniform, KL = LSE2 - mean_j s2_j - ln n_i.
    nq, nk, d = 4, 10, 3
    _, k1, q2, k2 = _inputs(nq, nk, d, seed=4)
    scale = 1.3
    for causal in (False, True):
        kl, _, _ = oracle.fwd(np.zeros_like(q2), k1, q2, k2, scale, causal)
        vis = _visible(nq, nk, causal)
        for i in range(nq):
            s2 = scale * (k2[vis[i]] @ q2[i])
            ref = scipy.special.logsumexp(s2) - s2.mean() - math.log(s2.size)
            assert kl[i] == pytest.approx(ref, rel=1e-11, abs=1e-14)


def test_single_visible_key(oracle_lib):
    # Causal row 0 with NQ = NK sees only key 0: KL = 0 and LSE_t = s_t,00.
    q1, k1, q2, k2 = _inputs(4, 4, 3, seed=5)
    kl, l1, l2 = oracle.fwd(q1, k1, q2, k2, 0.8, True)
    assert kl[0] == 0.0
    assert l1[0] == pytest.approx(0.8 * q1[0] @ k1[0], rel=1e-15)
    assert l2[0] == pytest.approx(0.8 * q2[0] @ k2[0], rel=1e-15)


def test_two_keys_bernoulli(oracle_lib):
    # Two visible keys: KL between Bernoulli(sigmoid(d1)) and Bernoulli(sigmoid(d2)).
    q1, k1, q2, k2 = _inputs(3, 2, 4, seed=6)
    scale = 0.6
    kl, _, _ = oracle.fwd(q1, k1, q2, k2, scale, False)
    for i in range(3):
        d1 = scale * q1[i] @ (k1[0] - k1[1])
        d2 = scale * q2[i] @ (k2[0] - k2[1])
        a, b = scipy.special.expit(d1), scipy.special.expit(d2)
        ref = a * math.log(a / b) + (1 - a) * math.log((1 - a) / (1 - b))
        assert kl[i] == pytest.approx(ref, rel=1e-11)


def test_identical_distributions_are_exact_zero(oracle_lib):
    q1, k1, _, _ = _inputs(6, 9, 4, seed=8)
    for causal in (False, True):
        out = oracle.bwd(q1, k1, q1, k1, 0.4, causal, np.full(6, 0.3))
        assert np.all(out["kl"] == 0.0)
        for k in ("dq1", "dq2", "dk1", "dk2"):
            assert np.all(out[k] == 0.0)


def test_kl_nonnegative_and_row_local(oracle_lib):
    q1, k1, q2, k2 = _inputs(16, 20, 6, seed=9, noise=1.5)
    for causal in (False, True):
        kl, _, _ = oracle.fwd(q1, k1, q2, k2, 0.5, causal)
        assert np.all(kl >= 0.0)
        # Row i depends only on Q1[i], Q2[i]: perturbing row 3 leaves the others unchanged.
        q1b = q1.copy()
        q1b[3] += 1.0
        kl2, _, _ = oracle.fwd(q1b, k1, q2, k2, 0.5, causal)
        mask = np.arange(16) != 3
        assert np.array_equal(kl[mask], kl2[mask]) and kl[3] != kl2[3]


def test_noncausal_key_permutation_invariance(oracle_lib):
    q1, k1, q2, k2 = _inputs(5, 12, 4, seed=10)
    perm = np.random.default_rng(0).permutation(12)
    a = oracle.fwd(q1, k1, q2, k2, 0.5, False)
    b = oracle.fwd(q1, k1[perm], q2, k2[perm], 0.5, False)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=1e-13, atol=1e-15)


def test_row_subset_matches_full(oracle_lib):
    q1, k1, q2, k2 = _inputs(9, 13, 4, seed=11)
    full = oracle.fwd(q1, k1, q2, k2, 0.5, True)
    rows = [8, 0, 5]
    sub = oracle.fwd(q1, k1, q2, k2, 0.5, True, rows=rows)
    for x, y in zip(full, sub):
        assert np.array_equal(x[rows], y)


# ---------------------------------------------------------------- gradients

def _loss(q1, k1, q2, k2, scale, causal, g):
    kl, _, _ = oracle.fwd(q1, k1, q2, k2, scale, causal)
    return float(np.dot(g, kl))


@pytest.mark.parametrize("nq,nk,d,causal", [(4, 6, 3, False), (4, 6, 3, True), (5, 5, 2, True), (6, 3, 4, False)])
def test_gradients_match_central_differences(oracle_lib, nq, nk, d, causal):
    q1, k1, q2, k2 = _inputs(nq, nk, d, seed=20 + nq * nk, noise=0.8)
    g = np.random.default_rng(2).uniform(-1.0, 1.0, nq)
    scale = 0.75
    out = oracle.bwd(q1, k1, q2, k2, scale, causal, g)
    args = [q1, k1, q2, k2]
    names = ["dq1", "dk1", "dq2", "dk2"]
    for which, name in enumerate(names):
        x = args[which]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            hstep = 1e-5 * max(1.0, abs(x[idx]))
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[which][idx] += hstep
            xm[which][idx] -= hstep
            fd[idx] = (_loss(*xp, scale, causal, g) - _loss(*xm, scale, causal, g)) / (2 * hstep)
        np.testing.assert_allclose(out[name], fd, rtol=1e-6, atol=1e-9, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd(oracle_lib, causal):
    nq, nk, d = 7, 9, 5
    q1, k1, q2, k2 = _inputs(nq, nk, d, seed=30, noise=0.6)
    g = np.random.default_rng(3).uniform(0.1, 1.0, nq)
    scale = 0.45
    out = oracle.bwd(q1, k1, q2, k2, scale, causal, g)
    ts = [torch.tensor(a, requires_grad=True) for a in (q1, k1, q2, k2)]
    vis = torch.from_numpy(_visible(nq, nk, causal))
    s1 = scale * ts[0] @ ts[1].T
    s2 = scale * ts[2] @ ts[3].T
    neg = torch.tensor(-1e300, dtype=torch.float64)  # finite: -inf poisons where() gradients
    lp1 = torch.log_softmax(torch.where(vis, s1, neg), -1)
    lp2 = torch.log_softmax(torch.where(vis, s2, neg), -1)
    zero = torch.zeros((), dtype=torch.float64)
    kl = torch.where(vis, lp1.exp() * (lp1 - lp2), zero).sum(-1)
    (torch.from_numpy(g) * kl).sum().backward()
    for t, name in zip(ts, ["dq1", "dk1", "dq2", "dk2"]):
        np.testing.assert_allclose(out[name], t.grad.numpy(), rtol=1e-11, atol=1e-13, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(oracle_lib, causal):
    # Adding c to every visible key of a row shifts its logits by scale*q.c: softmax is
    # unchanged, so sum_j dK_t[j] = 0 in every head.
    q1, k1, q2, k2 = _inputs(10, 12, 4, seed=40)
    g = np.random.default_rng(4).uniform(-1, 1, 10)
    out = oracle.bwd(q1, k1, q2, k2, 0.6, causal, g)
    for name in ("dk1", "dk2"):
        np.testing.assert_allclose(out[name].sum(0), 0.0, atol=1e-13)


def test_backward_is_linear_in_g_over_row_subsets(oracle_lib):
    q1, k1, q2, k2 = _inputs(8, 10, 3, seed=41)
    g = np.random.default_rng(5).uniform(-1, 1, 8)
    full = oracle.bwd(q1, k1, q2, k2, 0.5, True, g)
    a = oracle.bwd(q1, k1, q2, k2, 0.5, True, g[:3], rows=[0, 1, 2])
    b = oracle.bwd(q1, k1, q2, k2, 0.5, True, g[3:], rows=list(range(3, 8)))
    for name in ("dk1", "dk2"):
        np.testing.assert_allclose(a[name] + b[name], full[name], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(np.concatenate([a["dq1"], b["dq1"]]), full["dq1"], rtol=0, atol=0)


# ------------------------------------------------- the pages' online recurrence

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile,splits", [(1, 1), (3, 1), (5, 2), (4, 7), (64, 3)])
def test_online_recurrence_reaches_definition(oracle_lib, causal, tile, splits):
    # Streaming key tiles through (m1, l1, m2, l2, acc) and merging key chunks is exact:
    # it must agree with the definition to rounding, for any tiling, including empty chunks.
    q1, k1, q2, k2 = _inputs(9, 23, 4, seed=50, std=2.0, noise=1.0)
    scale = 0.8
    kl, l1, l2 = oracle.fwd(q1, k1, q2, k2, scale, causal)
    res = online.kl_online(q1, k1, q2, k2, scale, causal, tile=tile, splits=splits)
    np.testing.assert_allclose([r[0] for r in res], kl, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose([r[1] for r in res], l1, rtol=1e-13)
    np.testing.assert_allclose([r[2] for r in res], l2, rtol=1e-13)


def test_merge_identity_and_order(oracle_lib):
    rng = np.random.default_rng(60)
    s1, s2 = rng.standard_normal(40) * 3, rng.standard_normal(40) * 3
    a = online.run_row(s1[:17], s2[:17], [5, 9])
    b = online.run_row(s1[17:], s2[17:], [8])
    ab = online.merge([a, online.RowState(), b])
    ba = online.merge([b, a])
    whole = online.run_row(s1, s2, [13, 29])
    for st in (ab, ba):
        np.testing.assert_allclose(online.finish(st), online.finish(whole), rtol=1e-12)
