"""GPU parity of the backward pass (attn_bwd) against the fp64 oracle.

The GPU path runs attn_fwd, then attn_bwd on its O and lse; the oracle
differentiates the exact function.  Tolerance, from the arithmetic: the
products take dO, P and dS rounded to bf16 (relative error 2^-9 each) and D =
dO . O uses the forward's O, so each gradient is compared by its largest error
relative to its largest magnitude, max|dX - ref| <= 2e-2 * max|ref| (about ten
bf16 roundings), and by its root-mean-square error relative to the reference's,
<= 1e-2 (both magnitudes floored at 1e-4, for gradients that are exactly 0).
Small shapes are compared on every element; the full-size GQA case (B=2,
Hq=32, Hkv=8, N=8192, d=128, RoPE) on every (batch, KV head) pair at sampled
query and key rows.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")

MAX_REL = 2e-2
RMS_REL = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _grad_check(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), what
    # an exactly zero reference (one visible key: dQ = dK = 0) is measured
    # against an absolute floor of 1e-4
    scale = max(np.max(np.abs(ref)), 1e-4)
    mx = np.max(np.abs(got - ref)) / scale
    rms = math.sqrt(np.mean((got - ref) ** 2)) / max(math.sqrt(np.mean(ref ** 2)), 1e-4)
    say(f"{what}: max err / max|ref| = {mx:.3e} (tol {MAX_REL}), rms rel = {rms:.3e} (tol {RMS_REL})")
    assert mx <= MAX_REL and rms <= RMS_REL, what


def _run(q, k, v, do, causal, scale, rope_base=0.0):
    import torch
    dq_, dk_, dv_ = dev(q), dev(k), dev(v)
    o, lse = esd.fwd(dq_, dk_, dv_, causal=causal, scale=scale, rope_base=rope_base)
    g = esd.bwd(dq_, dk_, dv_, o, lse, dev(do), causal=causal, scale=scale, rope_base=rope_base)
    torch.cuda.synchronize()
    return tuple(host(x) for x in g)


def _inputs(seed, B, Hq, Hkv, Nq, Nk, d):
    q = W.normal((B, Hq, Nq, d), seed + 1, 1.0, "bf16")
    k = W.normal((B, Hkv, Nk, d), seed + 2, 1.0, "bf16")
    v = W.normal((B, Hkv, Nk, d), seed + 3, 1.0, "bf16")
    do = W.normal((B, Hq, Nq, d), seed + 4, 1.0, "f32")
    return q, k, v, do


SMALL = []
for d in (64, 128):
    for (Nq, Nk) in [(1, 1), (7, 7), (33, 33), (65, 65), (100, 130), (129, 300), (1, 200)]:
        for causal in (False, True):
            SMALL.append((d, Nq, Nk, causal))


@pytest.mark.parametrize("d,Nq,Nk,causal", SMALL)
def test_bwd_small(d, Nq, Nk, causal):
    q, k, v, do = _inputs(11000 + 3 * Nq + Nk + d, 1, 4, 2, Nq, Nk, d)
    scale = 1 / math.sqrt(d)
    got = _run(q, k, v, do, causal, scale)
    ref = oa.attention_bwd(q, k, v, do, causal=causal, scale=scale, dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"bwd {name} d={d} Nq={Nq} Nk={Nk} causal={causal}")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 1), (12, 4), (32, 8)])
def test_bwd_head_sharing(Hq, Hkv):
    q, k, v, do = _inputs(11200 + Hq, 1, Hq, Hkv, 300, 300, 128)
    got = _run(q, k, v, do, True, 0.0884)
    ref = oa.attention_bwd(q, k, v, do, causal=True, scale=0.0884, dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"bwd {name} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("d,Nq,Nk", [(128, 777, 777), (64, 777, 777), (128, 500, 1100),
                                     (64, 300, 1030)])
def test_bwd_causal_several_key_blocks(d, Nq, Nk):
    """Causal shapes with several 256-key blocks and 64-query tiles, where the
    waves of a key block skip the 32-query updates none of their keys is
    visible to at different points (bottom-right offset Nk - Nq included)."""
    q, k, v, do = _inputs(11600 + Nq + d, 1, 8, 2, Nq, Nk, d)
    scale = 1 / math.sqrt(d)
    got = _run(q, k, v, do, True, scale)
    ref = oa.attention_bwd(q, k, v, do, causal=True, scale=scale, dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"bwd {name} d={d} Nq={Nq} Nk={Nk} causal")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_rope(d):
    q, k, v, do = _inputs(11300 + d, 2, 8, 2, 150, 200, d)
    got = _run(q, k, v, do, True, 1 / math.sqrt(d), rope_base=10000.0)
    ref = oa.attention_bwd(q, k, v, do, causal=True, scale=1 / math.sqrt(d), rope_base=10000.0,
                           dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"bwd rope {name} d={d}")


@pytest.mark.parametrize("d,Nq,Nk", [(128, 500, 1100), (64, 700, 700)])
def test_bwd_rope_several_key_blocks(d, Nq, Nk):
    """RoPE with several 256-key blocks: dQ and dK are rotated back in the
    kernels' stores (dK from pairs split over neighbouring lanes), at query
    positions Nk - Nq + i and key positions j."""
    q, k, v, do = _inputs(11700 + Nq + d, 1, 8, 2, Nq, Nk, d)
    scale = 1 / math.sqrt(d)
    got = _run(q, k, v, do, True, scale, rope_base=10000.0)
    ref = oa.attention_bwd(q, k, v, do, causal=True, scale=scale, rope_base=10000.0,
                           dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"bwd rope {name} d={d} Nq={Nq} Nk={Nk}")


@pytest.mark.parametrize("d,Nq,Nk", [(128, 300, 100), (64, 129, 7)])
def test_bwd_more_queries_than_keys_unmasked(d, Nq, Nk):
    q, k, v, do = _inputs(11800 + Nq + d, 1, 8, 2, Nq, Nk, d)
    scale = 1 / math.sqrt(d)
    got = _run(q, k, v, do, False, scale)
    ref = oa.attention_bwd(q, k, v, do, causal=False, scale=scale, dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"bwd {name} unmasked Nq={Nq} > Nk={Nk} d={d}")


def test_bwd_deterministic():
    q, k, v, do = _inputs(11400, 1, 8, 2, 257, 257, 128)
    a = _run(q, k, v, do, True, 0.0884, 10000.0)
    b = _run(q, k, v, do, True, 0.0884, 10000.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_gqa_n8192_every_kv_head():
    """Causal GQA + RoPE 1e4, B=2 Hq=32 Hkv=8 N=8192 d=128: for each of the 16
    (batch, KV head) pairs, dQ on sampled query rows of its four query heads and
    dK, dV on sampled key rows (edges of the 256-key and 64-query blocks the
    kernels use, plus random rows drawn per pair)."""
    import torch
    w = W.WORKLOADS["gqa_rope_n8192"]
    q, k, v = W.fwd_inputs(w)
    do = W.normal((w.B, w.Hq, w.Nq, w.d), 11500, 1.0, "f32")
    say(f"bwd gqa_rope_n8192 shape: {w.note}")
    got = _run(q, k, v, do, True, w.scale, w.rope_base)
    N = w.Nq
    G = w.Hq // w.Hkv
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, N // 2, N - 257, N - 256, N - 65, N - 64,
             N - 33, N - 32, N - 2, N - 1]
    rng = np.random.default_rng(11501)
    for b in range(w.B):
        for g in range(w.Hkv):
            rows = np.unique(np.concatenate([fixed, rng.integers(0, N, 12)]))
            sq, sk, sv = oa.attention_bwd_rows(q, k, v, do, b, g, rows, rows, causal=True,
                                               scale=w.scale, rope_base=w.rope_base, dtype="bf16")
            tag = f"bwd gqa_rope_n8192 b={b} g={g}"
            _grad_check(got[0][b, g * G:(g + 1) * G][:, rows], sq, f"{tag} dq ({len(rows)} rows x {G} heads)")
            _grad_check(got[1][b, g, rows], sk, f"{tag} dk ({len(rows)} rows)")
            _grad_check(got[2][b, g, rows], sv, f"{tag} dv ({len(rows)} rows)")
    del got
    torch.cuda.empty_cache()


def test_bwd_group8_n8192_peaky():
    """Causal attention with 8 query heads per KV head (B=1, Hq=16, Hkv=2,
    N=8192, d=128), RoPE 5e5 and Q, K ~ N(0, 4^2), whose softmax rows are
    nearly one-hot, as in the long-context workload: 32 key blocks per KV head,
    each visiting the 8 heads of every query tile, with B * Hkv = 2 (not a
    multiple of the XCD count).  dQ on sampled query rows of all 16 heads, dK
    and dV on the same key rows, both KV heads."""
    import torch
    B, Hq, Hkv, N, d = 1, 16, 2, 8192, 128
    scale = 1 / math.sqrt(d)
    q = W.normal((B, Hq, N, d), 11601, 4.0, "bf16")
    k = W.normal((B, Hkv, N, d), 11602, 4.0, "bf16")
    v = W.normal((B, Hkv, N, d), 11603, 1.0, "bf16")
    do = W.normal((B, Hq, N, d), 11604, 1.0, "f32")
    say(f"bwd group of 8, peaky: B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} RoPE 5e5")
    got = _run(q, k, v, do, True, scale, 500000.0)
    G = Hq // Hkv
    fixed = [0, 1, 31, 32, 63, 64, 255, 256, 4095, 4096, N - 257, N - 256, N - 65, N - 64,
             N - 2, N - 1]
    rng = np.random.default_rng(11605)
    for g in range(Hkv):
        rows = np.unique(np.concatenate([fixed, rng.integers(0, N, 8)]))
        sq, sk, sv = oa.attention_bwd_rows(q, k, v, do, 0, g, rows, rows, causal=True,
                                           scale=scale, rope_base=500000.0, dtype="bf16")
        tag = f"bwd group of 8 g={g}"
        _grad_check(got[0][0, g * G:(g + 1) * G][:, rows], sq, f"{tag} dq ({len(rows)} rows x {G} heads)")
        _grad_check(got[1][0, g, rows], sk, f"{tag} dk ({len(rows)} rows)")
        _grad_check(got[2][0, g, rows], sv, f"{tag} dv ({len(rows)} rows)")
    del got
    torch.cuda.empty_cache()
