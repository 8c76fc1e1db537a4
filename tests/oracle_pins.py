"""Checks that tie the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something the pages or mathematics fix: a printed worked example, a closed
form, an invariant, brute force on tiny inputs, or an independent library
routine (torch's fp64 scaled_dot_product_attention and its bf16 conversion).
They are collected by ``test_oracle.py`` and re-run against deliberately broken
copies of the oracle by ``test_oracle_mutations.py``.

Page titles used below:
  [Breakdown]     "Transformer Architecture Breakdown" (airsota.com)
  [Deconstructed] "Transformer Architecture Deconstructed" (byronfinn.github.io)
  [Scratch]       "coding-interview attention from scratch" (arganzheng.life)
  [Evolution]     "Attention mechanisms: from alignment to efficient long context"
                  (fahimfaisal.info)
"""

from __future__ import annotations

import cmath
import math
import os

import numpy as np

import oracle.dense as oa

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def _rng(seed):
    return np.random.default_rng(seed)


def _bf16_via_torch(x64):
    """fp64 -> fp32 -> bf16 with torch's own conversions, back to fp64."""
    import torch
    t = torch.tensor(np.asarray(x64, np.float64))
    return t.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


def _rand_inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype, sigma=1.0):
    """Small random inputs already representable in ``dtype``."""
    r = _rng(seed)
    q = r.standard_normal((B, Hq, Nq, d)) * sigma
    k = r.standard_normal((B, Hkv, Nk, d)) * sigma
    v = r.standard_normal((B, Hkv, Nk, d))
    if dtype == "bf16":
        q, k, v = (_bf16_via_torch(x) for x in (q, k, v))
    elif dtype == "f32":
        q, k, v = (x.astype(np.float32).astype(np.float64) for x in (q, k, v))
    return q, k, v


# ------------------------------------------------------------ brute force
def _round_scalar(x, dtype):
    if dtype == "f64":
        return x
    if dtype == "f32":
        return float(np.float32(x))
    return float(_bf16_via_torch(np.array([x]))[0])


def _rot_complex(row, pos, base, dtype):
    """RoPE of one row as complex multiplication: pair t is x_2t + i x_2t+1,
    multiplied by e^(i pos theta_t), theta_t = base^(-2t/d) ([Breakdown] Key
    Topic 4 and section 3.1)."""
    d = len(row)
    out = []
    for t in range(d // 2):
        z = complex(row[2 * t], row[2 * t + 1]) * cmath.exp(1j * (pos * base ** (-2.0 * t / d)))
        out += [_round_scalar(z.real, dtype), _round_scalar(z.imag, dtype)]
    return out


def brute_attention(q, k, v, *, causal, scale, rope_base=0.0, dtype="f64", window=0):
    """Scalar-loop attention: for each query, exp-weights over visible keys.

    Visibility for t = Nq new queries over Nk keys follows [Scratch] 八 question 5
    (all earlier keys plus a lower triangle over the last Nq), query head h uses
    KV head from the repeat-interleave list of [Scratch] 三.4.
    """
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    group = [g for g in range(Hkv) for _ in range(Hq // Hkv)]
    o = np.zeros((B, Hq, Nq, d))
    lse = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = group[h]
            keys = [list(k[b, g, j]) for j in range(Nk)]
            if rope_base:
                keys = [_rot_complex(keys[j], j, rope_base, dtype) for j in range(Nk)]
            for i in range(Nq):
                qi = list(q[b, h, i])
                pos = Nk - Nq + i
                if rope_base:
                    qi = _rot_complex(qi, pos, rope_base, dtype)
                if window and causal:    # [Evolution] section 11: keys pos-w+1 .. pos
                    vis = list(range(max(0, pos - window + 1), pos + 1))
                elif window:             # both sides: pos-w+1 .. pos+w-1
                    vis = list(range(max(0, pos - window + 1), min(Nk, pos + window)))
                else:
                    vis = [j for j in range(Nk) if (not causal) or j <= pos]
                s = {j: scale * sum(qi[t] * keys[j][t] for t in range(d)) for j in vis}
                m = max(s.values())
                w = {j: math.exp(s[j] - m) for j in vis}
                z = sum(w.values())
                for t in range(d):
                    o[b, h, i, t] = sum(w[j] * v[b, g, j, t] for j in vis) / z
                lse[b, h, i] = m + math.log(z)
    return o, lse


# ------------------------------------------------------------ pins
def pin_softmax_worked_example():
    """[Scratch] 三.1 prints [0.090 0.245 0.665] for [1000, 1001, 1002]."""
    g = _golden("softmax_worked_example.txt")
    x = np.array([float(t) for t in g["input"]])
    want = np.array([float(t) for t in g["stable"]])
    got = oa.softmax(x[None, :])[0]
    assert np.all(np.round(got, int(g["decimals"][0])) == want), got
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(x) / np.exp(x).sum()
    assert all(t == "nan" for t in g["naive"]) and np.all(np.isnan(naive))
    assert abs(oa.logsumexp(x[None, :])[0] - (1002 + math.log(1 + math.exp(-1) + math.exp(-2)))) < 1e-12


def pin_softmax_shift_invariance():
    """Subtracting a constant from a row changes nothing ([Scratch] 三.1)."""
    x = _rng(1).standard_normal((16, 33)) * 3
    for c in (-7.5, 0.25, 40.0):
        # x + c itself rounds (ulp of 40 is 7e-15), so allow a few ulps
        assert np.max(np.abs(oa.softmax(x + c) - oa.softmax(x))) < 1e-13
        assert np.max(np.abs(oa.logsumexp(x + c) - (oa.logsumexp(x) + c))) < 1e-12


_SMALL = [
    # B, Hq, Hkv, Nq, Nk, d, causal, rope_base, dtype
    (1, 1, 1, 5, 5, 4, False, 0.0, "f64"),
    (1, 2, 2, 6, 6, 8, True, 0.0, "f32"),
    (2, 4, 2, 5, 7, 8, True, 10000.0, "bf16"),
    (1, 4, 1, 3, 8, 6, False, 100.0, "bf16"),
    (1, 3, 1, 7, 7, 4, True, 50.0, "f32"),
    (1, 2, 1, 1, 6, 8, True, 10.0, "bf16"),
]


def pin_brute_force_small():
    """Dense oracle = scalar loops (with complex-number RoPE) on tiny inputs."""
    for n, (B, Hq, Hkv, Nq, Nk, d, causal, base, dt) in enumerate(_SMALL):
        q, k, v = _rand_inputs(100 + n, B, Hq, Hkv, Nq, Nk, d, dt)
        scale = 1.0 / math.sqrt(d)
        o, lse = oa.attention(q, k, v, causal=causal, scale=scale, rope_base=base, dtype=dt)
        ob, lb = brute_attention(q, k, v, causal=causal, scale=scale, rope_base=base, dtype=dt)
        assert np.max(np.abs(o - ob)) < 1e-12, (n, np.max(np.abs(o - ob)))
        assert np.max(np.abs(lse - lb)) < 1e-12, (n, np.max(np.abs(lse - lb)))


def pin_torch_sdpa():
    """O equals torch's fp64 scaled_dot_product_attention (enable_gqa), the library
    routine [Scratch] 三.4 names for the comparison."""
    import torch
    import torch.nn.functional as F
    cases = [(2, 8, 2, 33, 33, 16, True), (1, 4, 4, 17, 40, 32, False),
             (1, 6, 1, 9, 9, 8, True), (2, 4, 2, 12, 30, 16, True)]
    for n, (B, Hq, Hkv, Nq, Nk, d, causal) in enumerate(cases):
        q, k, v = _rand_inputs(200 + n, B, Hq, Hkv, Nq, Nk, d, "f64")
        scale = 1.0 / math.sqrt(d)
        o, _ = oa.attention(q, k, v, causal=causal, scale=scale, dtype="f64")
        mask = None
        if causal:
            # visible iff j <= i + (Nk - Nq): bottom-right causal
            mask = torch.ones(Nq, Nk, dtype=torch.bool).tril(diagonal=Nk - Nq)
        ot = F.scaled_dot_product_attention(
            torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=mask,
            scale=scale, enable_gqa=True).numpy()
        assert np.max(np.abs(o - ot)) < 1e-12, (n, np.max(np.abs(o - ot)))


def pin_row_sums_and_mask():
    """Weights sum to 1; masked weights are exactly 0; a -1e9 fill gives the same
    weights as -inf ([Scratch] 三.2, [Breakdown] section 5 uses -1e9)."""
    r = _rng(3)
    q = r.standard_normal((9, 16))
    k = r.standard_normal((12, 16))
    qp = np.arange(9) + 3
    kp = np.arange(12)
    s, p = oa.scores_and_weights(q, k, scale=0.25, causal=True, q_pos=qp, k_pos=kp)
    assert np.max(np.abs(p.sum(-1) - 1)) < 1e-15
    masked = kp[None, :] > qp[:, None]
    assert masked.any() and np.all(p[masked] == 0.0)
    assert np.all(p[~masked] > 0)
    s9 = np.where(masked, -1e9, s)
    assert np.max(np.abs(oa.softmax(s9) - p)) == 0.0


def pin_causal_row0():
    """Causal query 0 sees only key 0: O_0 = V_0 and lse_0 = S_00, also with RoPE
    (position 0 is the identity rotation) ([Evolution] section 5 mask)."""
    for base in (0.0, 10000.0):
        q, k, v = _rand_inputs(7, 1, 2, 1, 10, 10, 8, "bf16")
        o, lse = oa.attention(q, k, v, causal=True, scale=0.3, rope_base=base, dtype="bf16")
        assert np.all(o[0, :, 0] == v[0, 0, 0])
        s00 = 0.3 * np.dot(q[0, :, 0], k[0, 0, 0].T)
        assert np.max(np.abs(lse[0, :, 0] - s00)) < 1e-14


def pin_uniform_scores():
    """Q = 0 makes every visible score equal: O_i is the mean of the visible V
    rows and lse_i = ln(number visible) (closed form of the definition)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 4, 2, 6, 11, 8
    _, k, v = _rand_inputs(8, B, Hq, Hkv, Nq, Nk, d, "f64")
    q = np.zeros((B, Hq, Nq, d))
    for causal in (False, True):
        o, lse = oa.attention(q, k, v, causal=causal, scale=0.5, rope_base=0.0, dtype="f64")
        for h in range(Hq):
            g = h // (Hq // Hkv)
            for i in range(Nq):
                n = (Nk - Nq + i + 1) if causal else Nk
                assert np.max(np.abs(o[0, h, i] - v[0, g, :n].mean(0))) < 1e-14
                assert abs(lse[0, h, i] - math.log(n)) < 1e-14


def pin_convex_hull():
    """Each output row is a convex combination of the visible V rows
    ([Deconstructed], multi-head section)."""
    q, k, v = _rand_inputs(9, 1, 2, 2, 16, 16, 8, "f64", sigma=3.0)
    o, _ = oa.attention(q, k, v, causal=True, scale=0.35, dtype="f64")
    for h in range(2):
        for i in range(16):
            vis = v[0, h, :i + 1]
            assert np.all(o[0, h, i] >= vis.min(0) - 1e-14)
            assert np.all(o[0, h, i] <= vis.max(0) + 1e-14)


def pin_gqa_equals_mha_repeat():
    """GQA equals MHA on K/V heads repeated H/H_kv times each, bitwise; H_kv = 1
    is MQA ([Scratch] 三.4, [Evolution] sections 8-9)."""
    for Hkv in (1, 2, 4):
        q, k, v = _rand_inputs(10 + Hkv, 2, 8, Hkv, 7, 9, 8, "bf16")
        o, lse = oa.attention(q, k, v, causal=True, scale=0.3, rope_base=500.0, dtype="bf16")
        kr = np.repeat(k, 8 // Hkv, axis=1)
        vr = np.repeat(v, 8 // Hkv, axis=1)
        o2, lse2 = oa.attention(q, kr, vr, causal=True, scale=0.3, rope_base=500.0, dtype="bf16")
        assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def pin_rope_relative():
    """Unrounded RoPE scores depend only on the position difference: q at t and k
    at t + 2 give the same product for t = 0, 3, 6 ([Scratch] 三.5), q at 3 with k
    at 7 equals q at 0 with k at 4 ([Breakdown] Key Topic 4); norms are kept."""
    r = _rng(11)
    d = 16
    q = r.standard_normal(d)
    k = r.standard_normal(d)
    dots = [np.dot(oa.rope(q[None], [t], 10000.0, "f64")[0],
                   oa.rope(k[None], [t + 2], 10000.0, "f64")[0]) for t in (0, 3, 6)]
    assert max(dots) - min(dots) < 1e-12
    a = np.dot(oa.rope(q[None], [3], 10000.0, "f64")[0], oa.rope(k[None], [7], 10000.0, "f64")[0])
    b = np.dot(q, oa.rope(k[None], [4], 10000.0, "f64")[0])
    assert abs(a - b) < 1e-12
    for p in (1, 17, 1000):
        x = oa.rope(q[None], [p], 10000.0, "f64")[0]
        assert abs(np.linalg.norm(x) - np.linalg.norm(q)) < 1e-12


def pin_rope_closed_form():
    """Pair 0 has theta_0 = 1, so (1, 0) at position p becomes (cos p, sin p) and
    (0, 1) becomes (-sin p, cos p): the counter-clockwise rotation matrix of
    [Breakdown] section 3.1.  Pair 1 of d = 4 turns by p / sqrt(base)."""
    for p in (0, 1, 2, 5, 1000):
        a = oa.rope(np.array([[1.0, 0.0, 1.0, 0.0]]), [p], 400.0, "f64")[0]
        b = oa.rope(np.array([[0.0, 1.0, 0.0, 1.0]]), [p], 400.0, "f64")[0]
        t1 = p / 20.0
        assert np.max(np.abs(a - [math.cos(p), math.sin(p), math.cos(t1), math.sin(t1)])) < 1e-13
        assert np.max(np.abs(b - [-math.sin(p), math.cos(p), -math.sin(t1), math.cos(t1)])) < 1e-13


def pin_rounding_vs_torch():
    """The rounding model equals torch's fp64 -> fp32 -> bf16 conversions,
    including values exactly halfway between two bf16 numbers."""
    r = _rng(12)
    x = np.concatenate([r.standard_normal(5000) * 10, r.standard_normal(100) * 1e-30])
    # exact halfway cases: an fp32 whose low 16 bits are 0x8000 lies halfway
    # between its two bf16 neighbours; upper halves with an even and an odd
    # last bit, both signs, normal exponents; and the fp32 values one step
    # either side of each tie
    hi = r.integers(0x0080, 0x7F00, 400).astype(np.uint32)
    hi[0::2] &= np.uint32(0xFFFE)
    hi[1::2] |= np.uint32(1)
    hi |= r.integers(0, 2, 400).astype(np.uint32) << np.uint32(15)
    ties = (hi << np.uint32(16)) | np.uint32(0x8000)
    near = np.concatenate([ties, ties - np.uint32(1), ties + np.uint32(1)])
    x = np.concatenate([x, near.view(np.float32).astype(np.float64)])
    assert np.array_equal(oa.round_to_dtype(x, "bf16"), _bf16_via_torch(x))
    assert np.array_equal(oa.round_to_dtype(x, "f32"), x.astype(np.float32).astype(np.float64))
    rot = oa.rope(r.standard_normal((4, 8)), np.arange(4), 10000.0, "bf16")
    assert np.array_equal(rot, _bf16_via_torch(rot))


def pin_decode_equals_last_causal_row():
    """A decode step over a cache of n keys equals row n-1 of causal prefill
    ([Scratch] 三.6 checks token-by-token decode against full causal attention)."""
    B, Hq, Hkv, N, d = 2, 4, 2, 13, 8
    q, k, v = _rand_inputs(13, B, Hq, Hkv, N, N, d, "f64")
    o, lse = oa.attention(q, k, v, causal=True, scale=0.4, dtype="f64")
    for n in (1, 5, 13):
        pad = np.full((B, Hkv, 20, d), np.nan)
        kc, vc = pad.copy(), pad.copy()
        kc[:, :, :n] = k[:, :, :n]
        vc[:, :, :n] = v[:, :, :n]
        od, ld = oa.decode(q[:, :, n - 1], kc, vc, np.array([n, n]), scale=0.4)
        # row n-1 of a causal prefill over the first n keys
        o2, l2 = oa.attention(q[:, :, :n], k[:, :, :n], v[:, :, :n], causal=True,
                              scale=0.4, dtype="f64")
        assert np.max(np.abs(od - o2[:, :, n - 1])) < 1e-14
        assert np.max(np.abs(ld - l2[:, :, n - 1])) < 1e-14
    assert np.max(np.abs(oa.decode(q[:, :, N - 1], k, v, np.array([N, N]), scale=0.4)[0]
                         - o[:, :, N - 1])) < 1e-14
    od, ld = oa.decode(q[:, :, 0], k, v, np.array([0, N]), scale=0.4)
    assert np.all(od[0] == 0) and np.all(np.isneginf(ld[0]))


def pin_score_std():
    """Unscaled q.k at d = 128 has std ~ 11.3 and 1 after the 1/sqrt(d) scale;
    with component variance sigma^2 the variance is d sigma^4 ([Breakdown]
    section 1.2, Key Topic 1)."""
    g = _golden("score_std.txt")
    d = int(g["d"][0])
    r = _rng(14)
    q = r.standard_normal((512, d))
    k = r.standard_normal((512, d))
    pos = np.arange(512)
    s1, _ = oa.scores_and_weights(q, k, scale=1.0, causal=False, q_pos=pos, k_pos=pos)
    s2, _ = oa.scores_and_weights(q, k, scale=1.0 / math.sqrt(d), causal=False, q_pos=pos, k_pos=pos)
    assert abs(np.std(s1) - float(g["unscaled_std"][0])) < 0.15, np.std(s1)
    assert abs(np.std(s2) - float(g["scaled_std"][0])) < 0.02, np.std(s2)
    s3, _ = oa.scores_and_weights(4 * q, 4 * k, scale=1.0 / math.sqrt(d), causal=False,
                                  q_pos=pos, k_pos=pos)
    assert abs(np.std(s3) - 16.0) < 0.3


def pin_lse_identity():
    """sum_j exp(S_ij - lse_i) over visible keys is 1 ([Scratch] 三.1: log-softmax
    is x minus logsumexp, and its exponentials sum to one)."""
    q, k, v = _rand_inputs(15, 1, 2, 1, 10, 14, 8, "f64", sigma=2.0)
    o, lse = oa.attention(q, k, v, causal=True, scale=0.5, dtype="f64")
    for h in range(2):
        s = 0.5 * q[0, h] @ k[0, 0].T
        vis = np.arange(14)[None, :] <= (np.arange(10) + 4)[:, None]
        tot = np.where(vis, np.exp(s - lse[0, h][:, None]), 0.0).sum(-1)
        assert np.max(np.abs(tot - 1)) < 1e-13


_WINDOWED = [
    # B, Hq, Hkv, Nq, Nk, d, causal, window, rope_base, dtype
    (1, 2, 1, 9, 9, 8, True, 3, 0.0, "f64"),
    (1, 4, 2, 6, 11, 8, True, 4, 100.0, "bf16"),
    (2, 2, 2, 7, 7, 4, False, 2, 0.0, "f32"),
    (1, 2, 1, 5, 12, 8, False, 5, 10.0, "bf16"),
]


def pin_window_brute_force_and_torch():
    """Windowed attention = scalar loops over the key range [p-w+1, p] (causal)
    or [p-w+1, p+w-1] ([Evolution] section 11), and = torch's fp64 SDPA with the
    explicit mask |i - j| < w (and j <= i)."""
    import torch
    import torch.nn.functional as F
    for n, (B, Hq, Hkv, Nq, Nk, d, causal, w, base, dt) in enumerate(_WINDOWED):
        q, k, v = _rand_inputs(300 + n, B, Hq, Hkv, Nq, Nk, d, dt)
        scale = 1.0 / math.sqrt(d)
        o, lse = oa.attention(q, k, v, causal=causal, scale=scale, rope_base=base, dtype=dt, window=w)
        ob, lb = brute_attention(q, k, v, causal=causal, scale=scale, rope_base=base, dtype=dt, window=w)
        assert np.max(np.abs(o - ob)) < 1e-12 and np.max(np.abs(lse - lb)) < 1e-12, n
        if base == 0.0:
            i = np.arange(Nq)[:, None] + (Nk - Nq)
            j = np.arange(Nk)[None, :]
            mask = np.abs(i - j) < w
            if causal:
                mask &= j <= i
            ot = F.scaled_dot_product_attention(
                torch.tensor(q), torch.tensor(k), torch.tensor(v), attn_mask=torch.tensor(mask),
                scale=scale, enable_gqa=True).numpy()
            assert np.max(np.abs(o - ot)) < 1e-12, n


def pin_window_special_cases():
    """w = 1 (causal) leaves each query its own position: O_i = V[p_i] exactly and
    lse_i = S[i, p_i]; a window at least as long as the keys changes nothing."""
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 6, 10, 8
    q, k, v = _rand_inputs(320, B, Hq, Hkv, Nq, Nk, d, "f64")
    o, lse = oa.attention(q, k, v, causal=True, scale=0.4, dtype="f64", window=1)
    for h in range(Hq):
        for i in range(Nq):
            p = Nk - Nq + i
            assert np.all(o[0, h, i] == v[0, 0, p])
            assert abs(lse[0, h, i] - 0.4 * np.dot(q[0, h, i], k[0, 0, p])) < 1e-13
    o1, l1 = oa.attention(q, k, v, causal=True, scale=0.4, dtype="f64", window=Nk)
    o2, l2 = oa.attention(q, k, v, causal=True, scale=0.4, dtype="f64")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def _padded_cache(k, v, lens, max_len, seed):
    """Caches [B,Hkv,max_len,d] holding k/v rows 0..lens[b]-1 and NaN after."""
    B, Hkv, _, d = k.shape
    kc = np.full((B, Hkv, max_len, d), np.nan)
    vc = np.full((B, Hkv, max_len, d), np.nan)
    for b, n in enumerate(lens):
        kc[b, :, :n] = k[b, :, :n]
        vc[b, :, :n] = v[b, :, :n]
    return kc, vc


def pin_decode_multi_against_page_mask():
    """T new tokens over a cache: torch's fp64 SDPA with the mask built as
    [Scratch] 八 question 5 states it, [all-True (T, len) | tril (T, T)], with
    the query rotated by complex multiplication at position len + t; and scalar
    loops (brute force) for the same rows."""
    import torch
    import torch.nn.functional as F
    B, Hq, Hkv, T, d, max_len = 3, 4, 2, 5, 8, 24
    lens = np.array([5, 12, 24])
    for base, dt in ((0.0, "f64"), (100.0, "bf16")):
        q, k, v = _rand_inputs(340 + int(base), B, Hq, Hkv, T, max_len, d, dt)
        kc, vc = _padded_cache(k, v, lens, max_len, 0)
        o, lse = oa.decode_multi(q, kc, vc, lens, scale=0.3, rope_base=base, dtype=dt)
        for b, n in enumerate(lens):
            hist = n - T
            mask = np.concatenate([np.ones((T, hist), bool), np.tril(np.ones((T, T), bool))], axis=1)
            qb = q[b].copy()
            if base:
                for h in range(Hq):
                    for t in range(T):
                        qb[h, t] = _rot_complex(list(q[b, h, t]), hist + t, base, dt)
            ot = F.scaled_dot_product_attention(
                torch.tensor(qb), torch.tensor(k[b, :, :n]), torch.tensor(v[b, :, :n]),
                attn_mask=torch.tensor(mask), scale=0.3, enable_gqa=True).numpy()
            assert np.max(np.abs(o[b] - ot)) < 1e-12, (b, base)
            ob, lb = brute_attention(qb[None], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                                     causal=True, scale=0.3, dtype="f64")
            assert np.max(np.abs(o[b] - ob[0])) < 1e-12 and np.max(np.abs(lse[b] - lb[0])) < 1e-12


def pin_decode_multi_incremental_and_short():
    """Decoding the T tokens one at a time (cache prefix of n - T + t + 1 rows)
    gives the same rows ([Scratch] 三.6: token-by-token decode = causal
    attention); T = 1 is the single-query decode; a sequence with fewer than T
    rows leaves its first tokens without keys (O = 0, lse = -inf)."""
    B, Hq, Hkv, T, d, max_len = 2, 4, 1, 4, 8, 16
    lens = np.array([2, 16])
    q, k, v = _rand_inputs(360, B, Hq, Hkv, T, max_len, d, "f64")
    kc, vc = _padded_cache(k, v, lens, max_len, 0)
    o, lse = oa.decode_multi(q, kc, vc, lens, scale=0.5, dtype="f64")
    for t in range(T):
        n_t = np.maximum(lens - T + t + 1, 0)
        od, ld = oa.decode(q[:, :, t], kc, vc, n_t, scale=0.5)
        assert np.max(np.abs(od - o[:, :, t])) < 1e-14
        assert np.array_equal(np.isneginf(ld), np.isneginf(lse[:, :, t]))
        fin = np.isfinite(ld)
        assert np.max(np.abs(ld[fin] - lse[:, :, t][fin])) < 1e-14
    assert np.all(o[0, :, :2] == 0) and np.all(np.isneginf(lse[0, :, :2]))
    assert np.all(np.isfinite(lse[0, :, 2:]))
    o1, l1 = oa.decode_multi(q[:, :, :1], kc, vc, lens, scale=0.5, dtype="f64")
    od, ld = oa.decode(q[:, :, 0], kc, vc, lens, scale=0.5)
    assert np.array_equal(o1[:, :, 0], od) and np.array_equal(l1[:, :, 0], ld)


class _PagePool:
    """The allocation procedure of [Evolution] section 20 and [Breakdown] Paged
    Attention, written as loops: a free list of physical blocks, a table per
    request that grows by one block whenever a position starts a new block,
    and each token's K/V written at kv[phys, :, offset, :]."""

    def __init__(self, num_blocks, block_size, Hkv, d, seed):
        self.free = list(_rng(seed).permutation(num_blocks))
        self.bs = block_size
        self.k = np.full((num_blocks, Hkv, block_size, d), np.nan)
        self.v = np.full((num_blocks, Hkv, block_size, d), np.nan)
        self.tables = {}

    def append_token(self, req, position, k_tok, v_tok):
        table = self.tables.setdefault(req, [])
        if position % self.bs == 0:
            table.append(self.free.pop())
        phys, off = table[position // self.bs], position % self.bs
        self.k[phys, :, off, :] = k_tok
        self.v[phys, :, off, :] = v_tok


def pin_paged_decode_equals_contiguous():
    """Tokens appended one by one into a shuffled block pool, then decoded
    through the block table, give exactly the contiguous-cache result (the
    attention arithmetic is unchanged, [Evolution] section 20), for block sizes
    that split sequences at different points; unused pool slots hold NaN."""
    B, Hq, Hkv, T, d, max_len = 3, 4, 2, 3, 8, 40
    lens = np.array([1, 17, 40])
    q, k, v = _rand_inputs(380, B, Hq, Hkv, T, max_len, d, "f64")
    kc, vc = _padded_cache(k, v, lens, max_len, 0)
    ref = oa.decode_multi(q, kc, vc, lens, scale=0.4, dtype="f64")
    for bs in (1, 4, 16):
        nblk = sum(-(-int(n) // bs) for n in lens) + 3
        pool = _PagePool(nblk, bs, Hkv, d, 390 + bs)
        for b, n in enumerate(lens):
            for p in range(n):
                pool.append_token(b, p, k[b, :, p], v[b, :, p])
        mb = max(len(t) for t in pool.tables.values())
        table = np.full((B, mb + 2), -1, dtype=np.int64)
        for b, t in pool.tables.items():
            table[b, :len(t)] = t
        got = oa.decode_paged(q, pool.k, pool.v, table, lens, block_size=bs, scale=0.4, dtype="f64")
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]), bs


def _torch_rope(x, positions, base):
    """RoPE in torch fp64 as complex multiplication ([Breakdown] Key Topic 4),
    differentiable, unrounded."""
    import torch
    d = x.shape[-1]
    th = torch.tensor([base ** (-2.0 * t / d) for t in range(d // 2)], dtype=torch.float64)
    ang = torch.tensor(positions, dtype=torch.float64)[:, None] * th[None, :]
    z = torch.view_as_complex(x.reshape(*x.shape[:-1], d // 2, 2).contiguous())
    return torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)).reshape(x.shape)


def pin_backward_against_autograd():
    """dQ, dK, dV equal torch's fp64 autograd through scaled_dot_product_attention
    (GQA by enable_gqa, causal by an explicit bottom-right mask, RoPE by a
    differentiable complex rotation; inputs already representable, so the
    oracle's rounding of rotated rows only matters with RoPE, where autograd
    sees unrounded rows: compared there with f64 rounding)."""
    import torch
    import torch.nn.functional as F
    cases = [(1, 2, 2, 5, 5, 8, False, 0.0, 0), (2, 4, 2, 6, 9, 8, True, 0.0, 0),
             (1, 4, 1, 7, 7, 4, True, 100.0, 0), (1, 2, 1, 8, 8, 8, True, 0.0, 3)]
    for n, (B, Hq, Hkv, Nq, Nk, d, causal, base, win) in enumerate(cases):
        q, k, v = _rand_inputs(400 + n, B, Hq, Hkv, Nq, Nk, d, "f64")
        do = _rng(410 + n).standard_normal((B, Hq, Nq, d))
        dq, dk, dv = oa.attention_bwd(q, k, v, do, causal=causal, scale=0.35, rope_base=base,
                                      dtype="f64", window=win)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        qq, kk = tq, tk
        if base:
            qq = _torch_rope(tq, np.arange(Nq) + Nk - Nq, base)
            kk = _torch_rope(tk, np.arange(Nk), base)
        mask = None
        if causal:
            i = np.arange(Nq)[:, None] + (Nk - Nq)
            j = np.arange(Nk)[None, :]
            m = j <= i
            if win:
                m &= i - j < win
            mask = torch.tensor(m)
        o = F.scaled_dot_product_attention(qq, kk, tv, attn_mask=mask, scale=0.35, enable_gqa=True)
        o.backward(torch.tensor(do))
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(got - ref.numpy())) < 1e-12, n


def pin_backward_finite_differences():
    """Central differences of L = sum(dO * O) in fp64 agree with the gradients
    (no library involved: the loss is the oracle's own forward)."""
    B, Hq, Hkv, Nq, Nk, d = 1, 2, 1, 4, 6, 4
    q, k, v = _rand_inputs(430, B, Hq, Hkv, Nq, Nk, d, "f64")
    do = _rng(431).standard_normal((B, Hq, Nq, d))

    def loss(q_, k_, v_):
        o, _ = oa.attention(q_, k_, v_, causal=True, scale=0.5, dtype="f64")
        return float(np.sum(o * do))

    dq, dk, dv = oa.attention_bwd(q, k, v, do, causal=True, scale=0.5, dtype="f64")
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        for idx in [(0, 0, 0, 0), (0, 0, 2, 3), (0, x.shape[1] - 1, x.shape[2] - 1, 1)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - g[idx]) < 1e-7 * max(1.0, abs(fd)), (idx, fd, g[idx])


def pin_backward_rows_equal_full():
    """The row-sampled backward (rowsum(P * dP) taken as dO . O) equals the full
    one on every sampled row, with and without RoPE, for groups of 2 and 4 query
    heads per KV head and fewer queries than keys (bottom-right positions)."""
    cases = [
        # B, Hq, Hkv, Nq, Nk, d, base, causal, (b, g), q rows, k rows
        (2, 4, 2, 9, 12, 8, 0.0, True, (1, 1), [0, 4, 8], [0, 3, 11]),
        (2, 4, 2, 9, 12, 8, 100.0, True, (1, 1), [0, 4, 8], [0, 3, 11]),
        (2, 4, 2, 9, 12, 8, 0.0, False, (1, 1), [0, 4, 8], [0, 3, 11]),
        (1, 8, 2, 7, 13, 8, 10000.0, True, (0, 1), [0, 3, 6], [0, 5, 6, 12]),
        (2, 8, 2, 6, 10, 16, 500.0, False, (1, 0), [1, 5], [0, 9]),
    ]
    for n, (B, Hq, Hkv, Nq, Nk, d, base, causal, (b, g), qr, kr) in enumerate(cases):
        q, k, v = _rand_inputs(440 + n, B, Hq, Hkv, Nq, Nk, d, "bf16")
        do = _rng(441 + n).standard_normal((B, Hq, Nq, d))
        dq, dk, dv = oa.attention_bwd(q, k, v, do, causal=causal, scale=0.3, rope_base=base,
                                      dtype="bf16")
        G = Hq // Hkv
        sq, sk, sv = oa.attention_bwd_rows(q, k, v, do, b, g, qr, kr, causal=causal, scale=0.3,
                                           rope_base=base, dtype="bf16")
        assert np.max(np.abs(sq - dq[b, g * G:(g + 1) * G][:, qr])) < 1e-12, n
        assert np.max(np.abs(sk - dk[b, g, kr])) < 1e-12, n
        assert np.max(np.abs(sv - dv[b, g, kr])) < 1e-12, n


def pin_bf16_bits_decoding():
    """Every one of the 65536 bf16 bit patterns is read as the value torch's
    bfloat16 dtype gives the same bits (NaN patterns as NaN), and fp32 arrays
    are widened unchanged.  Every GPU comparison reads its inputs this way."""
    import torch
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling NaN patterns warn on the cast
        got = oa._f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    x = _rng(16).standard_normal(1000).astype(np.float32)
    assert np.array_equal(oa._f64(x), x.astype(np.float64))


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
