"""Blocked online softmax and partial-state merge in fp64 (test infrastructure).

These follow the recurrence exactly as the pages state it, one query row at a
time, so the tests can pin the algebra the GPU kernels are built on:

* ``online_row``: "coding-interview attention from scratch", section 三.7 and
  "Attention mechanisms: from alignment to efficient long context", section 19:
  keep the running max m, the running sum l of exp(s - m) and the running
  weighted sum acc; when a block raises the max, multiply l and acc by
  exp(m_old - m_new) before adding the block; at the end O = acc / l.  The
  first block has m_old = -inf, whose factor is taken as 0.
* ``merge``: "Transformer Architecture Breakdown", section 4.2 and
  "Transformer Architecture Deconstructed", Online Softmax: two partial states
  (m1, d1, O1) and (m2, d2, O2) of disjoint key sets combine with
  m = max(m1, m2), d = d1 e^(m1-m) + d2 e^(m2-m),
  O = (d1 e^(m1-m) O1 + d2 e^(m2-m) O2) / d.  Applied pairwise, left to right,
  to any number of parts.  A part with no visible key (m = -inf) contributes 0.

Nothing here is imported by the GPU path; it models the algorithm only.
"""

from __future__ import annotations

import math

import numpy as np


def online_row(scores: np.ndarray, v: np.ndarray, block: int, *, rescale: bool = True):
    """O and (m, l) of one query row from its scores [n] (-inf = masked) and V [n, d].

    ``rescale=False`` drops the exp(m_old - m_new) correction: the defective
    variant the pages warn about, kept so a test can show that it is wrong.
    """
    scores = np.asarray(scores, np.float64)
    v = np.asarray(v, np.float64)
    m = -math.inf
    l = 0.0
    acc = np.zeros(v.shape[1])
    for s0 in range(0, len(scores), block):
        sb = scores[s0:s0 + block]
        m_new = max(m, float(sb.max()))
        if m_new == -math.inf:  # every key so far is masked
            continue
        if rescale:
            alpha = math.exp(m - m_new) if m > -math.inf else 0.0
        else:
            alpha = 1.0
        p = np.exp(sb - m_new)
        l = l * alpha + float(p.sum())
        acc = acc * alpha + p @ v[s0:s0 + block]
        m = m_new
    return acc / l, m, l


def partial(scores: np.ndarray, v: np.ndarray):
    """(m, d, O) of one key subset, computed densely: O normalised by d."""
    scores = np.asarray(scores, np.float64)
    m = float(scores.max()) if len(scores) else -math.inf
    if m == -math.inf:
        return m, 0.0, np.zeros(np.asarray(v).shape[1])
    e = np.exp(scores - m)
    d = float(e.sum())
    return m, d, (e @ np.asarray(v, np.float64)) / d


def merge(parts):
    """Combine partial states (m_i, d_i, O_i) of disjoint key sets, left to right."""
    m, d, o = parts[0]
    o = np.asarray(o, np.float64)
    for m2, d2, o2 in parts[1:]:
        mn = max(m, m2)
        if mn == -math.inf:
            continue
        a1 = d * math.exp(m - mn) if m > -math.inf else 0.0
        a2 = d2 * math.exp(m2 - mn) if m2 > -math.inf else 0.0
        dn = a1 + a2
        o = (a1 * o + a2 * np.asarray(o2, np.float64)) / dn
        m, d = mn, dn
    return m, d, o


def lse_of(m: float, d: float) -> float:
    """Natural-log logsumexp of a row from its partial state: m + ln d."""
    return m + math.log(d) if d > 0 else -math.inf
