"""GPU parity of the causal sliding window (attn_fwd_window) against the oracle.

The window follows "Attention mechanisms: from alignment to efficient long
context", section 11: a query at position p sees keys p-w+1 .. p.  Tolerances
as for attention without a window (bf16 max|dO| <= 1e-2, max|dlse| <= 1e-3;
fp32 1e-4).  Small shapes are compared element by element, with windows that
sit inside one tile, straddle tile edges, and cover every key; the full-size
cases (GQA N=8192 and N=32768 with w=4096) on sampled rows, including rows on
both sides of the point where the window starts to cut.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype):
    q = W.normal((B, Hq, Nq, d), seed + 1, 1.0, dtype)
    k = W.normal((B, Hkv, Nk, d), seed + 2, 1.0, dtype)
    v = W.normal((B, Hkv, Nk, d), seed + 3, 1.0, dtype)
    return q, k, v


def _run(q, k, v, window, scale, rope_base=0.0):
    import torch
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=True, scale=scale, rope_base=rope_base,
                     window=window)
    torch.cuda.synchronize()
    return host(o), host(lse)


CASES = []
for dtype in ("bf16", "f32"):
    for d in (64, 128):
        for (Nq, Nk) in [(65, 65), (129, 300), (300, 300)]:
            for w in (1, 5, 64, 100, 257):
                CASES.append((dtype, d, Nq, Nk, w))


@pytest.mark.parametrize("dtype,d,Nq,Nk,w", CASES)
def test_window_small(dtype, d, Nq, Nk, w):
    B, Hq, Hkv = 1, 4, 2
    q, k, v = _inputs(8000 + 7 * Nq + Nk + w, B, Hq, Hkv, Nq, Nk, d, dtype)
    scale = 1 / math.sqrt(d)
    o, lse = _run(q, k, v, w, scale)
    ro, rl = oa.attention(q, k, v, causal=True, scale=scale, dtype=dtype, window=w)
    check(o, lse, ro, rl, dtype, f"window {dtype} d={d} Nq={Nq} Nk={Nk} w={w}")


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (8, 1), (12, 4)])
@pytest.mark.parametrize("w", [3, 40, 200])
def test_window_head_sharing(Hq, Hkv, w):
    """MHA puts 256 rows (8 waves) of one head in a workgroup, so some waves
    see tiles wholly outside their window; GQA/MQA share tiles across heads."""
    q, k, v = _inputs(8300 + Hq + w, 1, Hq, Hkv, 600, 700, 128, "bf16")
    o, lse = _run(q, k, v, w, 0.0884)
    ro, rl = oa.attention(q, k, v, causal=True, scale=0.0884, dtype="bf16", window=w)
    check(o, lse, ro, rl, "bf16", f"window Hq={Hq} Hkv={Hkv} w={w}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_rope(dtype):
    q, k, v = _inputs(8400, 2, 8, 2, 200, 333, 128, dtype)
    o, lse = _run(q, k, v, 50, 0.0884, rope_base=10000.0)
    ro, rl = oa.attention(q, k, v, causal=True, scale=0.0884, rope_base=10000.0, dtype=dtype, window=50)
    check(o, lse, ro, rl, dtype, f"window+rope {dtype}")


def test_window_one_is_own_value_row():
    """w = 1 leaves each query only its own position: O_i = V[p_i] exactly."""
    q, k, v = _inputs(8500, 1, 4, 2, 100, 150, 64, "bf16")
    o, lse = _run(q, k, v, 1, 0.125)
    vf = W.as_f64(v, "bf16")
    qf, kf = W.as_f64(q, "bf16"), W.as_f64(k, "bf16")
    for h in range(4):
        for i in (0, 1, 63, 64, 99):
            p = 150 - 100 + i
            assert np.array_equal(o[0, h, i].astype(np.float64), vf[0, h // 2, p])
            assert abs(lse[0, h, i] - 0.125 * np.dot(qf[0, h, i], kf[0, h // 2, p])) < 1e-3


def test_window_covering_all_keys_equals_causal():
    import torch
    q, k, v = _inputs(8600, 1, 8, 2, 300, 300, 128, "bf16")
    a = _run(q, k, v, 300, 0.0884, 10000.0)
    b = _run(q, k, v, 10 ** 6, 0.0884, 10000.0)
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=True, scale=0.0884, rope_base=10000.0)
    torch.cuda.synchronize()
    c = (host(o), host(lse))
    for x in (a, b):
        assert np.array_equal(x[0], c[0]) and np.array_equal(x[1], c[1])


def test_window_rejects():
    import torch
    q, k, v = (dev(x) for x in _inputs(8700, 1, 2, 1, 8, 8, 64, "bf16"))
    with pytest.raises(esd.AttnError):
        esd.fwd(q, k, v, causal=True, window=-1)
    with pytest.raises(ValueError):
        esd.fwd(q, k, v, causal=False, window=4)
    torch.cuda.synchronize()


def _sampled_window(name, w, heads, n_random, seed):
    wl = W.WORKLOADS[name]
    q, k, v = W.fwd_inputs(wl)
    say(f"{name} shape with window {w}: {wl.note}")
    o, lse = _run(q, k, v, w, wl.scale, wl.rope_base)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    N = wl.Nq
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 63, 64, w - 2, w - 1, w, w + 1, w + 63, w + 64, N // 2, N - 65, N - 64, N - 1]
    kc = {}
    for (b, h) in heads:
        rows = np.unique(np.concatenate([fixed, rng.integers(0, N, n_random)]))
        ro, rl = oa.attention_rows(q, k, v, b, h, rows, causal=True, scale=wl.scale,
                                   rope_base=wl.rope_base, dtype=wl.dtype, window=w, _kcache=kc)
        check(o[b, h, rows], lse[b, h, rows], ro, rl, wl.dtype,
              f"{name} w={w} b={b} h={h} ({len(rows)} rows)")


def test_window_gqa_n8192_sampled():
    _sampled_window("gqa_rope_n8192", 4096, [(0, 0), (0, 5), (1, 31)], 40, 11)


def test_window_long_context_n32768_sampled():
    _sampled_window("gqa_rope_n32768", 4096, [(0, 0), (0, 9), (0, 63)], 40, 12)
