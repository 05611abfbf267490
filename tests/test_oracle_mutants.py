"""The oracle's pins catch planted mistakes.

Each case copies the C oracle's source, plants one plausible mistake (a
flipped sign, a dropped term, an off-by-one or misplaced causal mask, a
wrong operand, a dropped scale), builds it on the CPU and runs two pins that
do not use the oracle: the forward against a 50-digit mpmath evaluation of
the definition, and the gradients against torch autograd in fp64.  The real
oracle must pass both; every mutant must fail at least one.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import reference_mp

SRC = os.path.join(os.path.dirname(oracle.__file__), "streamkl_oracle.c")

# name -> (text in the oracle, replacement, which occurrence: 0 first, -1 last, None all)
MUTANTS = {
    "kl_sign": ("kl += p1 * (logp1 - logp2);", "kl += p1 * (logp2 - logp1);", None),
    "lse_without_max": ("return m + log(acc);", "return log(acc);", None),
    "causal_off_by_one": ("return j <= i + (nk - nq);", "return j < i + (nk - nq);", None),
    "causal_top_left": ("return j <= i + (nk - nq);", "return j <= i;", None),
    "teacher_scale_dropped": ("s1[j] = scale * dot(q1i, k1 + j * d, d);", "s1[j] = dot(q1i, k1 + j * d, d);", None),
    "student_wrong_keys": ("s2[j] = scale * dot(q2i, k2 + j * d, d);", "s2[j] = scale * dot(q2i, k1 + j * d, d);",
                           None),
    "dq_drops_kl_term": ("(logp1 - logp2 - kl[r])", "(logp1 - logp2)", 0),
    "dk_drops_kl_term": ("(logp1 - logp2 - kl[r])", "(logp1 - logp2)", -1),
    "dk_student_sign": ("double ds2 = g[r] * (p2 - p1);", "double ds2 = g[r] * (p1 - p2);", -1),
    "dq_student_sign": ("double ds2 = g[r] * (p2 - p1);", "double ds2 = g[r] * (p1 - p2);", 0),
    "dq_teacher_wrong_keys": ("dq1r[k] += ds1 * k1j[k];", "dq1r[k] += ds1 * k2j[k];", None),
    "dk_student_wrong_queries": ("dk2j[k] += ds2 * q2i[k];", "dk2j[k] += ds2 * q1i[k];", None),
    "dq_scale_dropped": ("dq1r[k] *= scale;", "dq1r[k] *= 1.0;", None),
}


def _mutate(text, old, new, which):
    n = text.count(old)
    assert n >= 1, f"mutation target not found: {old}"
    if which is None:
        return text.replace(old, new)
    pos = [i for i in range(len(text)) if text.startswith(old, i)][which]
    return text[:pos] + new + text[pos + len(old):]


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib_{name}.so"
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"])
    return oracle.configure(ctypes.CDLL(str(so)))


def _inputs(nq, nk, d, seed):
    rng = np.random.default_rng(seed)
    q1 = rng.standard_normal((nq, d))
    k1 = rng.standard_normal((nk, d))
    q2 = q1 + 0.6 * rng.standard_normal((nq, d))
    k2 = k1 + 0.6 * rng.standard_normal((nk, d))
    return q1, k1, q2, k2


def _forward_pin_holds():
    for nq, nk, d, causal in ((5, 7, 4, True), (4, 4, 3, False), (3, 8, 2, True)):
        q1, k1, q2, k2 = _inputs(nq, nk, d, seed=nq * 31 + nk)
        kl, l1, l2 = oracle.fwd(q1, k1, q2, k2, 0.7, causal)
        ref = reference_mp.kl_rows(q1.tolist(), k1.tolist(), q2.tolist(), k2.tolist(), 0.7, causal)
        for a, b in zip((kl, l1, l2), ref):
            if not np.allclose(a, np.array([float(x) for x in b]), rtol=1e-10, atol=1e-12):
                return False
    return True


def _gradient_pin_holds():
    for nq, nk, d, causal in ((7, 9, 5, True), (7, 9, 5, False), (6, 4, 3, False)):
        q1, k1, q2, k2 = _inputs(nq, nk, d, seed=50 + nq + nk)
        g = np.random.default_rng(nq).uniform(-1.0, 1.0, nq)
        scale = 0.45
        out = oracle.bwd(q1, k1, q2, k2, scale, causal, g)
        ts = [torch.tensor(a, requires_grad=True) for a in (q1, k1, q2, k2)]
        i = torch.arange(nq)[:, None]
        j = torch.arange(nk)[None, :]
        vis = (j <= i + (nk - nq)) if causal else torch.ones((nq, nk), dtype=torch.bool)
        neg = torch.tensor(-1e300, dtype=torch.float64)
        lp1 = torch.log_softmax(torch.where(vis, scale * ts[0] @ ts[1].T, neg), -1)
        lp2 = torch.log_softmax(torch.where(vis, scale * ts[2] @ ts[3].T, neg), -1)
        kl = torch.where(vis, lp1.exp() * (lp1 - lp2), torch.zeros((), dtype=torch.float64)).sum(-1)
        (torch.from_numpy(g) * kl).sum().backward()
        for t, name in zip(ts, ("dq1", "dk1", "dq2", "dk2")):
            if not np.allclose(out[name], t.grad.numpy(), rtol=1e-9, atol=1e-11):
                return False
    return True


@pytest.fixture()
def swap_oracle():
    saved = oracle._load()
    yield lambda lib: setattr(oracle, "_lib", lib)
    oracle._lib = saved


def test_real_oracle_passes_both_pins(oracle_lib):
    assert _forward_pin_holds()
    assert _gradient_pin_holds()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_are_caught(oracle_lib, swap_oracle, tmp_path, name):
    old, new, which = MUTANTS[name]
    src = _mutate(open(SRC).read(), old, new, which)
    swap_oracle(_build(src, tmp_path, name))
    caught = (not _forward_pin_holds()) or (not _gradient_pin_holds())
    assert caught, f"mutant {name} passes every pin"
