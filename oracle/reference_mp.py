"""High-precision brute force of attention KL -- TEST INFRASTRUCTURE ONLY.

Evaluates the textbook definition for tiny shapes with mpmath: build each
row's probabilities P_t,ij = exp(s_t,ij) / sum_k exp(s_t,ik) over the visible
keys, then KL_i = sum_j P1_ij * ln(P1_ij / P2_ij) as a ratio of probabilities
(not through logits), and LSE_t,i = ln sum_j exp(s_t,ij).  This is a second,
independent route to the quantity defined in the StreamKL abstract
(paperdance.org / fugumt.com) and is used to pin the C oracle.

Inputs are exact (Python floats or small integers); work precision is set by
`dps` decimal digits.
"""
from __future__ import annotations

from typing import List, Sequence

import mpmath


def _visible(i: int, j: int, nq: int, nk: int, causal: bool) -> bool:
    if j >= nk:
        return False
    return (not causal) or j <= i + (nk - nq)


def _logits(q: Sequence[Sequence[float]], k: Sequence[Sequence[float]], scale):
    return [[scale * mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(qi, kj))
             for kj in k] for qi in q]


def kl_rows(q1, k1, q2, k2, scale, causal: bool, dps: int = 50):
    """Return (kl, lse1, lse2) lists of mpf for every query row."""
    with mpmath.workdps(dps):
        scale = mpmath.mpf(scale)
        nq, nk = len(q1), len(k1)
        s1 = _logits(q1, k1, scale)
        s2 = _logits(q2, k2, scale)
        kls: List = []
        lse1s: List = []
        lse2s: List = []
        for i in range(nq):
            vis = [j for j in range(nk) if _visible(i, j, nq, nk, causal)]
            z1 = mpmath.fsum(mpmath.exp(s1[i][j]) for j in vis)
            z2 = mpmath.fsum(mpmath.exp(s2[i][j]) for j in vis)
            kl = mpmath.mpf(0)
            for j in vis:
                p1 = mpmath.exp(s1[i][j]) / z1
                p2 = mpmath.exp(s2[i][j]) / z2
                kl += p1 * mpmath.log(p1 / p2)
            kls.append(kl)
            lse1s.append(mpmath.log(z1))
            lse2s.append(mpmath.log(z2))
        return kls, lse1s, lse2s


def loss(q1, k1, q2, k2, scale, causal: bool, g, dps: int = 50):
    """L = sum_i g_i * KL_i at high precision (for finite differences)."""
    with mpmath.workdps(dps):
        kls, _, _ = kl_rows(q1, k1, q2, k2, scale, causal, dps)
        return mpmath.fsum(mpmath.mpf(gi) * kl for gi, kl in zip(g, kls))
