"""Dense fp64 definition of scaled-dot-product attention (test infrastructure).

Every function here follows the definition on the pages directly; nothing is
tiled, fused or reordered.  Inputs are the exact values of the stored arrays as
float64 (bf16 bits or fp32 widened without change).

Sources (page title, section):
* "Transformer Architecture Breakdown" (airsota.com), section 1.2: the attention
  formula softmax(Q K^T / sqrt(d_k) + M) V; Key Topic 5: the causal mask sets
  entries with j > i to minus infinity; section 3.1 and section 5: RoPE rotates
  adjacent pairs (x_2j, x_2j+1) by the angle m * theta_j.
* "coding-interview attention from scratch" (arganzheng.life), section 三.1:
  stable softmax and log-softmax via the row max; 三.2: masked scores become
  minus infinity so their weight is exactly zero; 三.4: query head h reads KV head
  h // (H / H_kv); 三.5: theta_i = base^(-2i/d), positions 0..T-1, even/odd pairs,
  V is not rotated; 三.6: a decode step attends the new query to every cached key
  without a mask; 八 question 5: with t new queries over len cached keys the
  visible set is [all of the cache | lower triangle], i.e. bottom-right aligned.
* "Attention mechanisms: from alignment to efficient long context"
  (fahimfaisal.info), Notation: n_q x n_k score matrix, h query heads, h_kv KV
  heads; section 9: the group index of a query head is h // (h / h_kv).

Readings where the pages are silent (each listed in the design notes):
* O and logsumexp are returned in float64 here; the GPU writes them as fp32.
* With RoPE on, the rotated Q and K are rounded back to the input dtype
  (fp64 -> fp32 -> bf16, each round-to-nearest-even) before the product, as a
  bf16 -> bf16 operator would; V is never rotated.
* theta_j = pow(base, -2j/d) for j = 0..d/2-1 with the C library ``pow``; the
  angle is the fp64 product position * theta_j; cos and sin are the C library's
  fp64 ``cos`` and ``sin`` (Python ``math``).
* Query i sits at position Nk - Nq + i, key j at position j; causal visibility
  is j <= Nk - Nq + i.
* Sliding window w ("Attention mechanisms: from alignment to efficient long
  context", section 11): a key is visible when |p_q - p_k| < w, and in a causal
  model also p_k <= p_q, so a causal query sees [p_q - w + 1, p_q].  w = 0
  means no window.
* logsumexp is the natural-log logsumexp of the visible scaled scores of a row.
"""

from __future__ import annotations

import math

import numpy as np


# ------------------------------------------------------------------ softmax
def softmax(x: np.ndarray) -> np.ndarray:
    """Row softmax with the row max subtracted first.

    "coding-interview attention from scratch", section 三.1: subtracting the row
    max leaves the result unchanged and keeps exp from overflowing.  Entries that
    are -inf get weight exactly 0.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def logsumexp(x: np.ndarray) -> np.ndarray:
    """Natural-log logsumexp of each row: m + log(sum exp(x - m)).

    Same page, section 三.1 (log-softmax is x minus this quantity).
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


# ------------------------------------------------------------------ rounding
def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype and return them as fp64.

    ``"f64"``: unchanged; ``"f32"``: fp64 -> fp32 (round to nearest even);
    ``"bf16"``: fp64 -> fp32 -> bf16, each step round to nearest even.
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f64":
        return x.copy()
    x32 = x.astype(np.float32)
    if dtype == "f32":
        return x32.astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    u = x32.view(np.uint32).astype(np.uint64)
    # keep the upper 16 bits after adding half an ulp, ties going to the even one
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    u32 = (u << 16).astype(np.uint32)
    return u32.view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ RoPE
_COS_SIN_CACHE: dict = {}


def rope_cos_sin(n_pos: int, d: int, base: float):
    """fp64 cos/sin of position * theta_j for positions 0..n_pos-1, j = 0..d/2-1.

    "Transformer Architecture Breakdown", section 3.1 (frequencies
    theta_j = base^(-2j/d)); "coding-interview attention from scratch", 三.5.
    Each value comes from ``math.cos`` / ``math.sin`` of the fp64 product.
    """
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    key = (int(n_pos), int(d), float(base))
    hit = _COS_SIN_CACHE.get(key)
    if hit is not None:
        return hit
    theta = [math.pow(base, -2.0 * j / d) for j in range(d // 2)]
    cos = np.empty((n_pos, d // 2), dtype=np.float64)
    sin = np.empty((n_pos, d // 2), dtype=np.float64)
    for j, th in enumerate(theta):
        ang = [float(p) * th for p in range(n_pos)]
        cos[:, j] = [math.cos(a) for a in ang]
        sin[:, j] = [math.sin(a) for a in ang]
    _COS_SIN_CACHE.clear()  # keep at most one table alive
    _COS_SIN_CACHE[key] = (cos, sin)
    return cos, sin


def rope(x: np.ndarray, positions: np.ndarray, base: float, dtype: str) -> np.ndarray:
    """Rotate adjacent pairs of the last axis and round to ``dtype``.

    x: [..., n, d] fp64 with row r of the n axis at ``positions[r]``.  Pair j of a
    row at position p becomes (x0 cos a - x1 sin a, x0 sin a + x1 cos a) with
    a = p * theta_j ("Transformer Architecture Breakdown", section 3.1 rotation
    matrix and section 5; "coding-interview attention from scratch", 三.5).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size and positions.min() < 0:
        raise ValueError("RoPE positions start at 0")
    cos_t, sin_t = rope_cos_sin(int(positions.max()) + 1, d, base)
    c = cos_t[positions]
    s = sin_t[positions]
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return round_to_dtype(out, dtype)


# ------------------------------------------------------------------ attention
def _f64(x) -> np.ndarray:
    """Exact fp64 values of an array slice; uint16 arrays are read as bf16 bits."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Query head h reads KV head h // (Hq / Hkv) (repeat-interleave grouping)."""
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def scores_and_weights(q_rows, k, *, scale, causal, q_pos, k_pos, window=0):
    """Scaled scores S (masked entries -inf) and softmax weights P for some rows.

    q_rows [r, d] at positions q_pos, k [n, d] at positions k_pos.  A key is
    visible to a query when not causal or when its position is <= the query's,
    and, with a window w > 0, when the two positions differ by less than w.
    """
    s = (np.asarray(q_rows, np.float64) @ np.asarray(k, np.float64).T) * scale
    kp = np.asarray(k_pos)[None, :]
    qp = np.asarray(q_pos)[:, None]
    vis = np.ones(s.shape, dtype=bool)
    if causal:
        vis &= kp <= qp
    if window:
        vis &= np.abs(qp - kp) < window
    if causal or window:
        s = np.where(vis, s, -np.inf)
    return s, softmax(s)


def attention_rows(q, k, v, b: int, h: int, rows, *, causal: bool, scale: float,
                   rope_base: float = 0.0, dtype: str = "bf16", window: int = 0, _kcache=None):
    """O [len(rows), d] and lse [len(rows)] for query rows of head (b, h).

    q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d]: fp32/fp64 arrays, or uint16 arrays of bf16
    bits; only the slices needed are widened to fp64.
    """
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if (causal or window or rope_base) and Nq > Nk:
        # bottom-right positions Nk - Nq + i would be negative for the first rows
        raise ValueError("causal, windowed or rotated attention needs Nq <= Nk")
    g = _kv_head(h, Hq, Hkv)
    rows = np.asarray(rows, dtype=np.int64)
    q_pos = rows + (Nk - Nq)
    k_pos = np.arange(Nk)
    qr = _f64(q[b, h, rows])
    kg = _f64(k[b, g])
    vg = _f64(v[b, g])
    if rope_base:
        qr = rope(qr, q_pos, rope_base, dtype)
        key = (b, g)
        if _kcache is not None and key in _kcache:
            kg = _kcache[key]
        else:
            kg = rope(kg, k_pos, rope_base, dtype)
            if _kcache is not None:
                _kcache.clear()
                _kcache[key] = kg
    o = np.empty((len(rows), d), dtype=np.float64)
    lse = np.empty(len(rows), dtype=np.float64)
    panel = max(1, (1 << 24) // max(Nk, 1))  # ~128 MB of fp64 scores per panel
    for s0 in range(0, len(rows), panel):
        sl = slice(s0, s0 + panel)
        s, p = scores_and_weights(qr[sl], kg, scale=scale, causal=causal,
                                  q_pos=q_pos[sl], k_pos=k_pos, window=window)
        o[sl] = p @ vg
        lse[sl] = logsumexp(s)
    return o, lse


def attention(q, k, v, *, causal: bool, scale: float, rope_base: float = 0.0,
              dtype: str = "bf16", window: int = 0):
    """Full O [B,Hq,Nq,d] and lse [B,Hq,Nq] (fp64) for every head and row."""
    B, Hq, Nq, d = q.shape
    o = np.empty((B, Hq, Nq, d), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    kc: dict = {}
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h] = attention_rows(
                q, k, v, b, h, np.arange(Nq), causal=causal, scale=scale,
                rope_base=rope_base, dtype=dtype, window=window, _kcache=kc)
    return o, lse


def decode(q, k_cache, v_cache, seq_lens, *, scale: float):
    """One-query decode over a contiguous cache (no mask, no RoPE).

    q [B,Hq,d]; caches [B,Hkv,max_len,d] (fp32/fp64, or uint16 bf16 bits);
    sequence b uses cache rows
    0..seq_lens[b]-1 ("coding-interview attention from scratch", 三.6).  A
    sequence of length 0 has no visible key: O = 0 and lse = -inf.
    """
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    o = np.zeros((B, Hq, d), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            s = (_f64(k_cache[b, g, :n]) @ _f64(q[b, h])) * scale
            p = softmax(s)
            o[b, h] = p @ _f64(v_cache[b, g, :n])
            lse[b, h] = logsumexp(s)
    return o, lse


def decode_multi(q, k_cache, v_cache, seq_lens, *, scale: float, rope_base: float = 0.0,
                 dtype: str = "bf16"):
    """T new queries per sequence over a contiguous cache.

    "coding-interview attention from scratch", 八 question 5: with t new tokens
    over len cached ones the score block is t x (len + t); the first len
    columns are all visible and the last t form a lower triangle.  Here the
    cache already holds the new tokens' K/V: sequence b has n = seq_lens[b]
    rows, the last T of them new, so new token t sits at position n - T + t and
    sees rows 0 .. n - T + t (the bottom-right causal rule).  Keys are stored
    already rotated (三.6); with rope_base > 0 the query is rotated at its own
    position and rounded to ``dtype``.  A token whose position is negative
    (n < T) sees no key: O = 0 and lse = -inf, as for a length-0 decode.

    q [B,Hq,T,d]; caches [B,Hkv,max_len,d]; returns O [B,Hq,T,d], lse [B,Hq,T].
    """
    B, Hq, T, d = q.shape
    Hkv = k_cache.shape[1]
    o = np.zeros((B, Hq, T, d), dtype=np.float64)
    lse = np.full((B, Hq, T), -np.inf, dtype=np.float64)
    for b in range(B):
        n = int(seq_lens[b])
        pos = np.arange(T) + (n - T)
        rows = np.nonzero(pos >= 0)[0]
        if len(rows) == 0:
            continue
        k_pos = np.arange(n)
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            qr = _f64(q[b, h, rows])
            if rope_base:
                qr = rope(qr, pos[rows], rope_base, dtype)
            s, p = scores_and_weights(qr, _f64(k_cache[b, g, :n]), scale=scale, causal=True,
                                      q_pos=pos[rows], k_pos=k_pos)
            o[b, h, rows] = p @ _f64(v_cache[b, g, :n])
            lse[b, h, rows] = logsumexp(s)
    return o, lse


def gather_paged(pool, block_table, n: int, b: int, block_size: int):
    """Logical cache rows 0..n-1 of sequence b from a paged pool.

    "Attention mechanisms: from alignment to efficient long context", section
    20: position p lives in physical block table[p // block_size] at offset
    p % block_size; "Transformer Architecture Breakdown" (Paged Attention)
    stores a block as kv_cache[phys, :, offset, :], i.e. the pool is
    [num_blocks, Hkv, block_size, d].  Returns [Hkv, n, d] as float64.
    """
    pos = np.arange(n)
    phys = np.asarray(block_table[b])[pos // block_size]
    rows = pool[phys, :, pos % block_size]          # [n, Hkv, d]
    return np.transpose(_f64(rows), (1, 0, 2))


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, *, block_size: int, scale: float,
                 rope_base: float = 0.0, dtype: str = "bf16"):
    """Multi-token decode over a paged KV cache.

    The attention is that of ``decode_multi`` (PagedAttention changes where K/V
    rows live, not the arithmetic: same section 20); each sequence's rows are
    first gathered through its block table.  q [B,Hq,T,d]; pools
    [num_blocks, Hkv, block_size, d]; block_table [B, max_blocks] int.
    """
    B, Hq, T, d = q.shape
    Hkv = k_pool.shape[1]
    n_max = max([int(n) for n in seq_lens] + [1])
    kc = np.zeros((B, Hkv, n_max, d))
    vc = np.zeros((B, Hkv, n_max, d))
    for b in range(B):
        n = int(seq_lens[b])
        kc[b, :, :n] = gather_paged(k_pool, block_table, n, b, block_size)
        vc[b, :, :n] = gather_paged(v_pool, block_table, n, b, block_size)
    return decode_multi(q, kc, vc, seq_lens, scale=scale, rope_base=rope_base, dtype=dtype)


def rope_transpose(g, positions, base: float):
    """Adjoint of the RoPE rotation: the rotation by the negative angle, no rounding.

    Carries a gradient taken with respect to rotated rows back to the rows
    before rotation (each pair rotation is orthogonal, so its transpose is its
    inverse).
    """
    g = np.asarray(g, np.float64)
    d = g.shape[-1]
    positions = np.asarray(positions, dtype=np.int64)
    cos_t, sin_t = rope_cos_sin(int(positions.max()) + 1, d, base)
    c, s = cos_t[positions], sin_t[positions]
    g0, g1 = g[..., 0::2], g[..., 1::2]
    out = np.empty_like(g)
    out[..., 0::2] = g0 * c + g1 * s
    out[..., 1::2] = -g0 * s + g1 * c
    return out


def attention_bwd(q, k, v, do, *, causal: bool, scale: float, rope_base: float = 0.0,
                  dtype: str = "bf16", window: int = 0):
    """Gradients dQ, dK, dV (fp64) of L = sum(dO * O) for O = attention(q, k, v).

    The pages state only that the backward pass recomputes the score tiles
    from the saved per-row statistics ("Transformer Architecture
    Deconstructed", recomputation strategy; "Attention mechanisms: from
    alignment to efficient long context", section 19); the gradient itself is
    that of the function ``attention`` defines, written out per head:
      P = softmax(S), S = scale * Q K^T + M     (masked entries have P = 0)
      dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
      dQ = scale * dS K,  dK = scale * dS^T Q.
    Query heads that share a KV head add their dK and dV.  With RoPE, Q and K
    enter as rotated and rounded rows; the rounding is taken as the identity
    and the rotation's transpose carries dQ and dK back to the unrotated rows.
    q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d], do [B,Hq,Nq,d] (any real dtype, or uint16
    bf16 bits); returns dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d].
    """
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    if (causal or window or rope_base) and Nq > Nk:
        raise ValueError("causal, windowed or rotated attention needs Nq <= Nk")
    q_pos = np.arange(Nq) + (Nk - Nq)
    k_pos = np.arange(Nk)
    dq = np.zeros((B, Hq, Nq, d))
    dk = np.zeros((B, Hkv, Nk, d))
    dv = np.zeros((B, Hkv, Nk, d))
    for b in range(B):
        for h in range(Hq):
            g = _kv_head(h, Hq, Hkv)
            qh, kh, vh = _f64(q[b, h]), _f64(k[b, g]), _f64(v[b, g])
            doh = _f64(do[b, h])
            if rope_base:
                qh = rope(qh, q_pos, rope_base, dtype)
                kh = rope(kh, k_pos, rope_base, dtype)
            _, p = scores_and_weights(qh, kh, scale=scale, causal=causal, q_pos=q_pos,
                                      k_pos=k_pos, window=window)
            dv[b, g] += p.T @ doh
            dp = doh @ vh.T
            ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
            dqh = scale * (ds @ kh)
            dkh = scale * (ds.T @ qh)
            if rope_base:
                dqh = rope_transpose(dqh, q_pos, rope_base)
                dkh = rope_transpose(dkh, k_pos, rope_base)
            dq[b, h] = dqh
            dk[b, g] += dkh
    return dq, dk, dv


def attention_bwd_rows(q, k, v, do, b: int, g: int, q_rows, k_rows, *, causal: bool,
                       scale: float, rope_base: float = 0.0, dtype: str = "bf16"):
    """Selected rows of the backward pass for KV head g of batch b.

    Same gradient as ``attention_bwd``, evaluated only where asked: dQ for the
    query rows ``q_rows`` of every query head that reads KV head g, and dK, dV
    for the key rows ``k_rows`` of KV head g.  rowsum(P * dP) is taken as
    dO . O, the identity that follows from O = P V, with O and lse from
    ``attention_rows`` over every query row of those heads.  Returns
    dq [G, len(q_rows), d], dk [len(k_rows), d], dv [len(k_rows), d].
    """
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    G = Hq // Hkv
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    q_pos = np.arange(Nq) + (Nk - Nq)
    k_pos = np.arange(Nk)
    kg, vg = _f64(k[b, g]), _f64(v[b, g])
    if rope_base:
        kg = rope(kg, k_pos, rope_base, dtype)
    dq = np.zeros((G, len(q_rows), d))
    dk = np.zeros((len(k_rows), d))
    dv = np.zeros((len(k_rows), d))
    kc: dict = {}
    for hh in range(G):
        h = g * G + hh
        o, lse = attention_rows(q, k, v, b, h, np.arange(Nq), causal=causal, scale=scale,
                                rope_base=rope_base, dtype=dtype, _kcache=kc)
        doh = _f64(do[b, h])
        dvec = np.sum(doh * o, axis=-1)
        qh = _f64(q[b, h])
        if rope_base:
            qh = rope(qh, q_pos, rope_base, dtype)
        # dQ rows: P row, dP row, dS row
        s_r, _ = scores_and_weights(qh[q_rows], kg, scale=scale, causal=causal,
                                    q_pos=q_pos[q_rows], k_pos=k_pos)
        p_r = np.exp(s_r - lse[q_rows][:, None])
        ds_r = p_r * (doh[q_rows] @ vg.T - dvec[q_rows][:, None])
        dq_h = scale * (ds_r @ kg)
        dq[hh] = rope_transpose(dq_h, q_pos[q_rows], rope_base) if rope_base else dq_h
        # dK, dV rows: the score columns of the selected keys over every query
        s_c, _ = scores_and_weights(qh, kg[k_rows], scale=scale, causal=causal,
                                    q_pos=q_pos, k_pos=k_pos[k_rows])
        p_c = np.exp(s_c - lse[:, None])
        dv += p_c.T @ doh
        ds_c = p_c * (doh @ vg[k_rows].T - dvec[:, None])
        dk += scale * (ds_c.T @ qh)
    if rope_base:
        dk = rope_transpose(dk, k_pos[k_rows], rope_base)
    return dq, dk, dv
