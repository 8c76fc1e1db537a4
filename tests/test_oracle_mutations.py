"""Plant plausible mistakes in a copy of the oracle and check that a pin fails.

Each mutation swaps one oracle function for a broken version (dropped scale,
wrong rotation sign, wrong pairing, wrong head mapping, mask off by one, ...).
If every pin still passed, the pins would not be able to tell the oracle from
that mistake.  All of this runs on the CPU against the oracle only.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
from oracle_pins import ALL_PINS

_orig_scores = oa.scores_and_weights
_orig_rope = oa.rope
_orig_lse = oa.logsumexp


def _scores_no_scale(q_rows, k, *, scale, causal, q_pos, k_pos, window=0):
    return _orig_scores(q_rows, k, scale=1.0, causal=causal, q_pos=q_pos, k_pos=k_pos, window=window)


def _scores_strict(q_rows, k, *, scale, causal, q_pos, k_pos, window=0):
    # mask off by one: j < i instead of j <= i (the diagonal hidden)
    s = (np.asarray(q_rows) @ np.asarray(k).T) * scale
    if causal:
        vis = np.asarray(k_pos)[None, :] < np.asarray(q_pos)[:, None]
        s = np.where(vis, s, -np.inf)
    with np.errstate(invalid="ignore"):
        return s, oa.softmax(s)


def _scores_top_left(q_rows, k, *, scale, causal, q_pos, k_pos, window=0):
    # causal aligned at the top-left corner instead of the bottom-right
    q_pos = np.asarray(q_pos) - (np.asarray(q_pos).min() if len(q_pos) else 0)
    return _orig_scores(q_rows, k, scale=scale, causal=causal, q_pos=q_pos, k_pos=k_pos, window=window)


def _scores_transposed(q_rows, k, *, scale, causal, q_pos, k_pos, window=0):
    s = (np.asarray(q_rows) @ np.asarray(k).T) * scale
    if s.shape[0] == s.shape[1]:
        s = s.T.copy()
    if causal:
        vis = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
        s = np.where(vis, s, -np.inf)
    return s, oa.softmax(s)


def _rope_neg(x, positions, base, dtype):
    return _orig_rope(x, -np.asarray(positions), base, dtype) if False else \
        _rope_generic(x, positions, base, dtype, sign=-1)


def _rope_generic(x, positions, base, dtype, sign=1, half=False, expo=2.0):
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    pos = np.asarray(positions, np.float64)
    th = np.array([math.pow(base, -expo * j / d) for j in range(d // 2)])
    a = sign * pos[:, None] * th[None, :]
    c, s = np.cos(a), np.sin(a)
    if half:
        x0, x1 = x[..., : d // 2], x[..., d // 2:]
    else:
        x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    r0, r1 = x0 * c - x1 * s, x0 * s + x1 * c
    if half:
        out[..., : d // 2], out[..., d // 2:] = r0, r1
    else:
        out[..., 0::2], out[..., 1::2] = r0, r1
    return oa.round_to_dtype(out, dtype)


def _rope_half(x, positions, base, dtype):
    return _rope_generic(x, positions, base, dtype, half=True)


def _rope_theta(x, positions, base, dtype):
    return _rope_generic(x, positions, base, dtype, expo=1.0)


def _rope_unrounded(x, positions, base, dtype):
    return _orig_rope(x, positions, base, "f64")


def _lse_no_max(x):
    x = np.asarray(x, np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    return np.log(np.sum(np.exp(x - m), axis=-1))


def _lse_log2(x):
    return _orig_lse(x) / math.log(2.0)


def _kv_mod(h, Hq, Hkv):
    return h % Hkv


def _round_truncate(x, dtype):
    x = np.asarray(x, np.float64)
    if dtype != "bf16":
        return x.astype(np.float32).astype(np.float64) if dtype == "f32" else x.copy()
    u = x.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def _scores_window_le(q_rows, k, *, scale, causal, q_pos, k_pos, window=0):
    # window off by one: |i - j| <= w instead of < w
    return _orig_scores(q_rows, k, scale=scale, causal=causal, q_pos=q_pos, k_pos=k_pos,
                        window=window + 1 if window else 0)


_orig_decode_multi = oa.decode_multi


def _decode_multi_hides_self(q, k_cache, v_cache, seq_lens, **kw):
    # each new token misses its own row: positions n - T + t - 1
    return _orig_decode_multi(q, k_cache, v_cache, np.asarray(seq_lens) - 1, **kw)


_orig_gather = oa.gather_paged


def _gather_swapped(pool, block_table, n, b, block_size):
    # block index and offset swapped: table[p % bs], offset p // bs
    pos = np.arange(n)
    phys = np.asarray(block_table[b])[np.minimum(pos % block_size, np.asarray(block_table).shape[1] - 1)]
    rows = pool[phys, :, np.minimum(pos // block_size, pool.shape[2] - 1)]
    return np.transpose(np.asarray(rows, np.float64), (1, 0, 2))


def _rope_transpose_forward(g, positions, base):
    # rotates forward instead of by the negative angle
    return _rope_generic(g, positions, base, "f64")


def _bwd_without_rowsum(q, k, v, do, *, causal, scale, rope_base=0.0, dtype="bf16", window=0):
    # dS = P * dP, the softmax Jacobian's rowsum term dropped
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    dq = np.zeros((B, Hq, Nq, d))
    dk = np.zeros((B, Hkv, Nk, d))
    dv = np.zeros((B, Hkv, Nk, d))
    qp, kp = np.arange(Nq) + Nk - Nq, np.arange(Nk)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            qh, kh, vh = (np.asarray(x, np.float64) for x in (q[b, h], k[b, g], v[b, g]))
            if rope_base:
                qh, kh = oa.rope(qh, qp, rope_base, dtype), oa.rope(kh, kp, rope_base, dtype)
            _, p = oa.scores_and_weights(qh, kh, scale=scale, causal=causal, q_pos=qp, k_pos=kp,
                                         window=window)
            dv[b, g] += p.T @ do[b, h]
            ds = p * (do[b, h] @ vh.T)
            dqh, dkh = scale * ds @ kh, scale * ds.T @ qh
            if rope_base:
                dqh, dkh = oa.rope_transpose(dqh, qp, rope_base), oa.rope_transpose(dkh, kp, rope_base)
            dq[b, h] = dqh
            dk[b, g] += dkh
    return dq, dk, dv


_orig_f64 = oa._f64


def _f64_as_fp16(x):
    # bf16 bits misread as IEEE half precision
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return x.view(np.float16).astype(np.float64)
    return _orig_f64(x)


def _bwd_rows_wrong_group(q, k, v, do, b, g, q_rows, k_rows, **kw):
    # the query heads of the next KV head summed into this one's dK, dV
    Hkv = k.shape[1]
    return _orig_bwd_rows(q, k, v, do, b, (g + 1) % Hkv, q_rows, k_rows, **kw)


_orig_bwd_rows = oa.attention_bwd_rows

def _rope_query_at_row_index(x, positions, base, dtype):
    # queries rotated at their row index i instead of their position Nk - Nq + i
    # (key positions start at 0 and are left alone)
    p = np.asarray(positions)
    if p.size and p.min() > 0:
        p = p - p.min()
    return _orig_rope(x, p, base, dtype)


_orig_round = oa.round_to_dtype


def _softmax_no_max(x):
    # the naive form: exp of the raw scores (overflows for large scores)
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        return e / np.sum(e, axis=-1, keepdims=True)


def _round_ties_away(x, dtype):
    # bf16 rounding with ties away from zero instead of to the even neighbour
    if dtype != "bf16":
        return _orig_round(x, dtype)
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + 0x8000) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


MUTATIONS = {
    "rope_query_at_row_index": ("rope", _rope_query_at_row_index),
    "softmax_no_max_shift": ("softmax", _softmax_no_max),
    "bf16_ties_away_from_zero": ("round_to_dtype", _round_ties_away),
    "bf16_bits_read_as_fp16": ("_f64", _f64_as_fp16),
    "bwd_rows_wrong_group": ("attention_bwd_rows", _bwd_rows_wrong_group),
    "bwd_rope_not_transposed": ("rope_transpose", _rope_transpose_forward),
    "bwd_dropped_rowsum": ("attention_bwd", _bwd_without_rowsum),
    "paged_index_swapped": ("gather_paged", _gather_swapped),
    "decode_multi_hides_self": ("decode_multi", _decode_multi_hides_self),
    "window_off_by_one": ("scores_and_weights", _scores_window_le),
    "dropped_scale": ("scores_and_weights", _scores_no_scale),
    "mask_off_by_one": ("scores_and_weights", _scores_strict),
    "causal_top_left": ("scores_and_weights", _scores_top_left),
    "transposed_scores": ("scores_and_weights", _scores_transposed),
    "rope_wrong_sign": ("rope", _rope_neg),
    "rope_rotate_half": ("rope", _rope_half),
    "rope_wrong_theta": ("rope", _rope_theta),
    "rope_not_rounded": ("rope", _rope_unrounded),
    "lse_dropped_max": ("logsumexp", _lse_no_max),
    "lse_log2": ("logsumexp", _lse_log2),
    "gqa_mod_mapping": ("_kv_head", _kv_mod),
    "bf16_truncation": ("round_to_dtype", _round_truncate),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    oa._COS_SIN_CACHE.clear()
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin detects the mutation {name}"
