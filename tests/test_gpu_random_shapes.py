"""Seeded random shapes through attn_fwd / attn_fwd_window against the oracle:
head dims 64 and 128, groups of 1-8 query heads per KV head (powers of two and
not), ragged Nq <= Nk, causal or unmasked, sliding windows, RoPE bases, bf16 and
fp32 inputs.  Each draw is small enough for the oracle; the cases are fixed by
the seed, printed before they run."""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


def _draw(n, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        Nk = int(rng.integers(1, 700))
        causal = bool(rng.random() < 0.7)
        rope = float(rng.choice([0.0, 10000.0, 500000.0])) if causal else 0.0
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 700))
        window = int(rng.integers(1, Nk + 40)) if causal and rng.random() < 0.4 else 0
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        B = int(rng.choice([1, 2]))
        cases.append((i, dtype, d, B, Hkv * G, Hkv, Nq, Nk, causal, window, rope))
    return cases


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("case", _draw(32), ids=lambda c: f"r{c[0]}")
def test_random_shape(case):
    import torch
    i, dtype, d, B, Hq, Hkv, Nq, Nk, causal, window, rope = case
    what = (f"case {i}: {dtype} d={d} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} "
            f"window={window} rope={rope}")
    say(what)
    q = W.normal((B, Hq, Nq, d), 30000 + 4 * i, 1.5, dtype)
    k = W.normal((B, Hkv, Nk, d), 30001 + 4 * i, 1.5, dtype)
    v = W.normal((B, Hkv, Nk, d), 30002 + 4 * i, 1.0, dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=causal, scale=scale, rope_base=rope,
                     window=window)
    torch.cuda.synchronize()
    ro, rl = oa.attention(q, k, v, causal=causal, scale=scale, rope_base=rope, dtype=dtype,
                          window=window)
    check(host(o), host(lse), ro, rl, dtype, what)


MAX_REL = 2e-2   # gradients: max error over the largest reference magnitude
RMS_REL = 1e-2   # and RMS error over the reference's RMS (the backward tests' bar)


def _draw_bwd(n, seed=2027):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 3, 4]))
        Nk = int(rng.integers(1, 300))
        causal = bool(rng.random() < 0.7)
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 300))
        rope = float(rng.choice([0.0, 10000.0])) if Nq <= Nk else 0.0
        cases.append((i, d, int(rng.choice([1, 2])), Hkv * G, Hkv, Nq, Nk, causal, rope))
    return cases


@pytest.mark.parametrize("case", _draw_bwd(12), ids=lambda c: f"b{c[0]}")
def test_random_backward(case):
    import torch
    i, d, B, Hq, Hkv, Nq, Nk, causal, rope = case
    what = f"bwd case {i}: d={d} B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} causal={causal} rope={rope}"
    say(what)
    q = W.normal((B, Hq, Nq, d), 31000 + 5 * i, 1.0, "bf16")
    k = W.normal((B, Hkv, Nk, d), 31001 + 5 * i, 1.0, "bf16")
    v = W.normal((B, Hkv, Nk, d), 31002 + 5 * i, 1.0, "bf16")
    do = W.normal((B, Hq, Nq, d), 31003 + 5 * i, 1.0, "f32")
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = dev(q), dev(k), dev(v)
    o, lse = esd.fwd(tq, tk, tv, causal=causal, scale=scale, rope_base=rope)
    got = esd.bwd(tq, tk, tv, o, lse, dev(do), causal=causal, scale=scale, rope_base=rope)
    torch.cuda.synchronize()
    refs = oa.attention_bwd(q, k, v, do, causal=causal, scale=scale, rope_base=rope, dtype="bf16")
    for name, g, r in zip(("dq", "dk", "dv"), got, refs):
        g = np.asarray(host(g), np.float64)
        assert np.all(np.isfinite(g)), f"{what} {name}"
        top = max(np.max(np.abs(r)), 1e-4)
        mx = np.max(np.abs(g - r)) / top
        rms = math.sqrt(np.mean((g - r) ** 2)) / max(math.sqrt(np.mean(r ** 2)), 1e-4)
        say(f"  {name}: max err / max|ref| = {mx:.3e}, rms rel = {rms:.3e}")
        assert mx <= MAX_REL and rms <= RMS_REL, f"{what} {name}"


def _draw_dec(n, seed=2028):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8]))
        T = int(rng.choice([1, 2, 3, 4]))
        B = int(rng.integers(1, 5))
        max_len = int(rng.integers(1, 3000))
        lens = rng.integers(0, max_len + 1, B).astype(np.int32)
        rope = float(rng.choice([0.0, 10000.0]))
        paged = bool(rng.random() < 0.5)
        bs = int(rng.choice([16, 64, 256])) if paged else 0
        cases.append((i, d, B, Hkv * G, Hkv, T, max_len, lens, rope, bs))
    return cases


@pytest.mark.parametrize("case", _draw_dec(16), ids=lambda c: f"d{c[0]}")
def test_random_decode(case):
    """Multi-token decode over contiguous or paged caches (lengths from 0)."""
    import torch
    i, d, B, Hq, Hkv, T, max_len, lens, rope, bs = case
    what = (f"decode case {i}: d={d} B={B} Hq={Hq} Hkv={Hkv} T={T} max_len={max_len} "
            f"lens={lens.tolist()} rope={rope} block={bs}")
    say(what)
    q = W.normal((B, Hq, T, d), 32000 + 5 * i, 1.0, "bf16")
    scale = 1.0 / math.sqrt(d)
    if bs:
        nblk = [(int(n) + bs - 1) // bs for n in lens]
        mb = max(1, max(nblk))
        nb = sum(nblk) + 3
        perm = np.random.default_rng(32001 + i).permutation(nb)
        table = np.full((B, mb), -1, np.int32)
        pos = 0
        for b in range(B):
            table[b, :nblk[b]] = perm[pos:pos + nblk[b]]
            pos += nblk[b]
        kp = W.normal((nb, Hkv, bs, d), 32002 + 5 * i, 1.0, "bf16")
        vp = W.normal((nb, Hkv, bs, d), 32003 + 5 * i, 1.0, "bf16")
        o, lse = esd.decode_paged(dev(q), dev(kp), dev(vp), dev(table), dev(lens), scale=scale,
                                  rope_base=rope)
        torch.cuda.synchronize()
        ro, rl = oa.decode_paged(q, kp, vp, table, lens, block_size=bs, scale=scale,
                                 rope_base=rope, dtype="bf16")
    else:
        kc = W.normal((B, Hkv, max_len, d), 32002 + 5 * i, 1.0, "bf16")
        vc = W.normal((B, Hkv, max_len, d), 32003 + 5 * i, 1.0, "bf16")
        o, lse = esd.decode_multi(dev(q), dev(kc), dev(vc), dev(lens), scale=scale, rope_base=rope)
        torch.cuda.synchronize()
        ro, rl = oa.decode_multi(q, kc, vc, lens, scale=scale, rope_base=rope, dtype="bf16")
    go, gl = host(o), host(lse)
    dead = np.isneginf(rl)  # a token before any key: O = 0, lse = -inf
    assert np.array_equal(np.isneginf(gl), dead) and np.all(go[dead] == 0), what
    if (~dead).any():
        check(go[~dead], gl[~dead], ro[~dead], rl[~dead], "bf16", what)


# A wider sweep from other seeds: 300 forward and window shapes, 60 backward,
# 100 decode (every case runs the same checks as above); then longer sequences.
@pytest.mark.parametrize("case", _draw(300, seed=9101), ids=lambda c: f"w{c[0]}")
def test_random_shape_wide(case):
    test_random_shape(case)


@pytest.mark.parametrize("case", _draw_bwd(60, seed=9102), ids=lambda c: f"w{c[0]}")
def test_random_backward_wide(case):
    test_random_backward(case)


@pytest.mark.parametrize("case", _draw_dec(100, seed=9103), ids=lambda c: f"w{c[0]}")
def test_random_decode_wide(case):
    test_random_decode(case)


def _draw_long(n, seed):
    """Longer sequences (700-3000 keys): many row blocks and tiles, ragged tails."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4, 8]))
        Nk = int(rng.integers(700, 3000))
        causal = bool(rng.random() < 0.7)
        rope = float(rng.choice([0.0, 10000.0, 500000.0])) if causal else 0.0
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 3000))
        window = int(rng.integers(1, Nk + 40)) if causal and rng.random() < 0.4 else 0
        dtype = "f32" if rng.random() < 0.15 else "bf16"
        cases.append((i, dtype, d, 1, Hkv * G, Hkv, Nq, Nk, causal, window, rope))
    return cases


def _draw_bwd_long(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([1, 2]))
        G = int(rng.choice([1, 2, 4]))
        Nk = int(rng.integers(300, 1500))
        causal = bool(rng.random() < 0.7)
        Nq = int(rng.integers(1, Nk + 1)) if causal else int(rng.integers(1, 1500))
        rope = float(rng.choice([0.0, 10000.0])) if causal else 0.0
        cases.append((i, d, 1, Hkv * G, Hkv, Nq, Nk, causal, rope))
    return cases


@pytest.mark.parametrize("case", _draw_long(120, seed=9201), ids=lambda c: f"l{c[0]}")
def test_random_shape_long(case):
    test_random_shape(case)


@pytest.mark.parametrize("case", _draw_bwd_long(20, seed=9202), ids=lambda c: f"l{c[0]}")
def test_random_backward_long(case):
    test_random_backward(case)
