"""Blocked online softmax and partial-state merge in fp64 (test infrastructure).

These model, one query row at a time, the algebra the GPU kernels are built
on, so the tests can pin it:

* ``partial``: the state (m, d, O) of one subset of keys, formed densely: m is
  the largest score, d the sum of exp(s - m), O the d-normalised weighted sum
  of the value rows.
* ``merge``: "Transformer Architecture Breakdown", section 4.2 and
  "Transformer Architecture Deconstructed", Online Softmax: two states of
  disjoint key sets combine by bringing both sums to the larger max,
  m = max(m1, m2), d = d1 e^(m1-m) + d2 e^(m2-m),
  O = (d1 e^(m1-m) O1 + d2 e^(m2-m) O2) / d; applied pairwise, left to right,
  to any number of parts.  A part with no visible key (m = -inf) contributes
  nothing.
* ``online_row``: the streaming form ("coding-interview attention from
  scratch", section 三.7; "Attention mechanisms: from alignment to efficient
  long context", section 19) as a left fold: the row's keys arrive in blocks,
  and the running state absorbs each block's partial state with ``merge``.
  The factor e^(m_old - m_new) that ``merge`` applies to the running state is
  the rescale of the running sum and accumulator the pages describe.
* ``online_row_uncorrected``: the same stream with that factor left out (each
  block weighted against the running max, earlier sums never brought up to
  date) -- the defect the pages warn about, kept so a test can show it wrong.

Nothing here is imported by the GPU path; it models the algorithm only.
"""

from __future__ import annotations

import math

import numpy as np


def online_row(scores: np.ndarray, v: np.ndarray, block: int):
    """O and (m, l) of one query row from its scores [n] (-inf = masked) and V [n, d],
    reading the keys ``block`` at a time and folding each block's partial
    state into the running one."""
    scores = np.asarray(scores, np.float64)
    v = np.asarray(v, np.float64)
    state = (-math.inf, 0.0, np.zeros(v.shape[1]))
    for s0 in range(0, len(scores), block):
        state = merge([state, partial(scores[s0:s0 + block], v[s0:s0 + block])])
    m, l, o = state
    return o, m, l


def online_row_uncorrected(scores: np.ndarray, v: np.ndarray, block: int):
    """The stream without the correction factor: every block's weights are taken
    against the largest score seen so far, but what was summed before a larger
    score arrived is not scaled down to it.  Exact only while the largest score
    of the row sits in the first block."""
    scores = np.asarray(scores, np.float64)
    v = np.asarray(v, np.float64)
    top = -math.inf
    total = 0.0
    weighted = np.zeros(v.shape[1])
    for s0 in range(0, len(scores), block):
        blk = scores[s0:s0 + block]
        top = max(top, float(blk.max()))
        if top == -math.inf:
            continue
        w = np.exp(blk - top)
        total += float(w.sum())
        weighted += w @ v[s0:s0 + block]
    return weighted / total, top, total


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
