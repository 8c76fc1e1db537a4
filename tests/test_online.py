"""The blocked online-softmax recurrence and the partial merge (fp64, CPU).

Pins: "coding-interview attention from scratch", section 三.7 reports that the
blocked form with block 2 over 7 keys matches dense attention to 1e-16, and
question 4 of section 八 says dropping the rescale is only right when every
block's max equals the first block's.  The merge rule is the two-block formula
of "Transformer Architecture Breakdown", section 4.2.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import oracle.online as ol


def _dense(s, v):
    p = oa.softmax(s[None, :])[0]
    return p @ v, oa.logsumexp(s[None, :])[0]


@pytest.mark.parametrize("n,block", [(7, 2), (1, 4), (64, 64), (65, 64), (129, 16), (200, 7)])
def test_online_equals_dense(n, block):
    r = np.random.default_rng(n * 31 + block)
    s = r.standard_normal(n) * 6
    v = r.standard_normal((n, 5))
    o, m, l = ol.online_row(s, v, block)
    od, lsed = _dense(s, v)
    assert np.max(np.abs(o - od)) < 1e-12
    assert abs(ol.lse_of(m, l) - lsed) < 1e-12


def test_page_example_block2_seven_keys():
    r = np.random.default_rng(7)
    d = 4
    q = r.standard_normal(d)
    k = r.standard_normal((7, d))
    v = r.standard_normal((7, d))
    s = k @ q / math.sqrt(d)
    o, _, _ = ol.online_row(s, v, 2)
    assert np.max(np.abs(o - _dense(s, v)[0])) < 1e-15


def test_online_masked_prefix_blocks():
    # causal rows can start with a block whose keys are all masked
    s = np.array([-np.inf, -np.inf, -np.inf, 0.5, 2.0, -np.inf, 1.0])
    v = np.arange(14, dtype=float).reshape(7, 2)
    o, m, l = ol.online_row(s, v, 3)
    od, lsed = _dense(s, v)
    assert np.max(np.abs(o - od)) < 1e-14 and abs(ol.lse_of(m, l) - lsed) < 1e-14


def test_no_rescale_is_wrong_unless_first_block_holds_max():
    r = np.random.default_rng(3)
    v = r.standard_normal((8, 3))
    rising = np.array([0.0, 0.1, 0.2, 0.3, 3.0, 3.1, 3.2, 3.3])
    o_bad, _, _ = ol.online_row_uncorrected(rising, v, 4)
    assert np.max(np.abs(o_bad - _dense(rising, v)[0])) > 1e-3
    first = np.array([5.0, 0.1, 0.2, 0.3, 1.0, 1.1, 1.2, 1.3])
    o_ok, _, _ = ol.online_row_uncorrected(first, v, 4)
    assert np.max(np.abs(o_ok - _dense(first, v)[0])) < 1e-14


@pytest.mark.parametrize("cuts", [[3], [1, 2, 9], [5, 5, 5], [0, 4], [10, 11]])
def test_merge_equals_single_pass(cuts):
    r = np.random.default_rng(sum(cuts) + 1)
    n = 12
    s = r.standard_normal(n) * 4
    v = r.standard_normal((n, 6))
    edges = [0] + sorted(cuts) + [n]
    parts = [ol.partial(s[a:b], v[a:b]) for a, b in zip(edges[:-1], edges[1:])]
    m, d, o = ol.merge(parts)
    od, lsed = _dense(s, v)
    assert np.max(np.abs(o - od)) < 1e-13
    assert abs(ol.lse_of(m, d) - lsed) < 1e-13


def test_merge_associative():
    r = np.random.default_rng(5)
    parts = [ol.partial(r.standard_normal(5) * 3, r.standard_normal((5, 4))) for _ in range(4)]
    a = ol.merge([ol.merge(parts[:2]), ol.merge(parts[2:])])
    b = ol.merge(parts)
    assert abs(a[0] - b[0]) == 0 and abs(a[1] - b[1]) < 1e-13
    assert np.max(np.abs(a[2] - b[2])) < 1e-14
