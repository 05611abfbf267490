"""fp64 model of the pages' online algorithm -- TEST INFRASTRUCTURE ONLY.

The StreamKL forward (gist.science "Formulacion Online (Paso hacia
adelante)") keeps five running scalars per query row while it streams key
tiles: running maxima m1, m2 of the two logit rows, unnormalised exponential
sums l1, l2, and an accumulator acc of the P1-weighted logit difference.  At
the end it emits the row objective acc/l1 + LSE2 - LSE1 with
LSE_t = m_t + log l_t.  This module steps through that recurrence tile by
tile, in the pages' notation, so that tests can show it reaches the
definition (the C oracle) for any tiling.

The pages also split the key dimension across thread blocks for short query
counts (gist.science "Variante Split-K") but print no merge rule; `merge`
combines per-chunk states with the log-sum-exp rescaling that the recurrence
itself uses between tiles (a reading, stated here): the maximum is taken over
chunks, and each chunk's (l, acc) are rescaled by exp(m_chunk - m_max) before
summing; a chunk with no visible key is the identity.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterable, List, Sequence

import numpy as np


@dataclass
class RowState:
    m1: float = -math.inf
    l1: float = 0.0
    m2: float = -math.inf
    l2: float = 0.0
    acc: float = 0.0


def _rescale(m_old: float, m_new: float) -> float:
    if m_old == -math.inf:
        return 0.0
    return math.exp(m_old - m_new)


def update(st: RowState, s1: np.ndarray, s2: np.ndarray) -> RowState:
    """Fold one tile of visible scaled logits (1-D arrays) into the row state."""
    if s1.size == 0:
        return st
    m1n = max(st.m1, float(np.max(s1)))
    m2n = max(st.m2, float(np.max(s2)))
    a1 = _rescale(st.m1, m1n)
    a2 = _rescale(st.m2, m2n)
    e1 = np.exp(s1 - m1n)
    e2 = np.exp(s2 - m2n)
    return RowState(
        m1=m1n,
        l1=a1 * st.l1 + float(np.sum(e1)),
        m2=m2n,
        l2=a2 * st.l2 + float(np.sum(e2)),
        acc=a1 * st.acc + float(np.sum(e1 * (s1 - s2))),
    )


def finish(st: RowState):
    """(KL, LSE1, LSE2) from a final row state: KL = acc/l1 + LSE2 - LSE1."""
    lse1 = st.m1 + math.log(st.l1)
    lse2 = st.m2 + math.log(st.l2)
    return st.acc / st.l1 + lse2 - lse1, lse1, lse2


def merge(states: Iterable[RowState]) -> RowState:
    """Combine row states of disjoint key chunks (order-independent)."""
    states = [s for s in states if s.l1 > 0.0]
    if not states:
        return RowState()
    M1 = max(s.m1 for s in states)
    M2 = max(s.m2 for s in states)
    out = RowState(m1=M1, m2=M2)
    for s in states:
        w1 = math.exp(s.m1 - M1)
        w2 = math.exp(s.m2 - M2)
        out.l1 += w1 * s.l1
        out.acc += w1 * s.acc
        out.l2 += w2 * s.l2
    return out


def row_logits(q1, k1, q2, k2, scale: float, i: int, causal: bool):
    """Scaled logits of row i over its visible keys, in key order (fp64)."""
    nq, nk = q1.shape[0], k1.shape[0]
    last = nk if not causal else min(nk, i + (nk - nq) + 1)
    s1 = scale * (k1[:last] @ q1[i])
    s2 = scale * (k2[:last] @ q2[i])
    return s1, s2


def run_row(s1: np.ndarray, s2: np.ndarray, boundaries: Sequence[int]) -> RowState:
    """Stream one row's logits through tiles whose end offsets are `boundaries`."""
    st = RowState()
    start = 0
    for end in list(boundaries) + [s1.size]:
        end = min(end, s1.size)
        if end > start:
            st = update(st, s1[start:end], s2[start:end])
            start = end
    return st


def kl_online(q1, k1, q2, k2, scale: float, causal: bool, tile: int = 64,
              splits: int = 1) -> List[tuple]:
    """Per-row (KL, LSE1, LSE2) by the online recurrence over `tile`-key tiles,
    with the key range cut into `splits` chunks that are merged at the end."""
    q1, k1, q2, k2 = (np.asarray(a, dtype=np.float64) for a in (q1, k1, q2, k2))
    nk = k1.shape[0]
    chunk = -(-nk // splits)
    out = []
    for i in range(q1.shape[0]):
        s1, s2 = row_logits(q1, k1, q2, k2, scale, i, causal)
        parts = []
        for c in range(splits):
            lo, hi = c * chunk, min((c + 1) * chunk, s1.size)
            if hi <= lo:
                parts.append(RowState())
                continue
            b = list(range(tile, hi - lo, tile))
            parts.append(run_row(s1[lo:hi], s2[lo:hi], b))
        out.append(finish(merge(parts)))
    return out
