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
