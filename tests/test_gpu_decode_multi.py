"""GPU parity of multi-token decode (attn_decode_multi) against the oracle.

T new tokens per sequence over a cache that already holds their K/V; token t
sits at position n - T + t and sees cache rows 0 .. n - T + t
("coding-interview attention from scratch", 八 question 5).  Tolerances as for
single-token decode (bf16 inputs: max|dO| <= 1e-2, max|dlse| <= 1e-3).  The
lengths cover sequences shorter than T (tokens without keys: O = 0, lse =
-inf), the 32-key batch, 128-key wave and 1024-key chunk edges, and chunks in
which only the last new tokens see a key; the caches hold NaN past each
length, so a read past the end would show.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")

LENS = np.array([0, 1, 2, 3, 5, 31, 33, 127, 1023, 1024, 1025, 1027, 2047, 2048, 2049, 2100, 3000,
                 4097], dtype=np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _inputs(lens, Hq, Hkv, T, max_len, d, seed):
    w = W.WORKLOADS["decode_b32"]
    _, kc, vc = W.decode_inputs(w, lens, Hq=Hq, Hkv=Hkv, max_len=max_len, d=d, seed_base=seed)
    q = W.normal((len(lens), Hq, T, d), seed + 7, 1.0, "bf16")
    return q, kc, vc


def _run(q, kc, vc, lens, scale, rope_base=0.0):
    import torch
    o, lse = esd.decode_multi(dev(q), dev(kc), dev(vc), dev(lens), scale=scale, rope_base=rope_base)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _check_rows(o, lse, ro, rl, what):
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), what
    assert np.all(o[dead] == 0), what
    live = ~dead
    check(o[live], lse[live], ro[live], rl[live], "bf16", what)


@pytest.mark.parametrize("Hq,Hkv,T", [(8, 8, 2), (8, 8, 3), (32, 8, 4), (32, 8, 5), (16, 2, 2),
                                      (32, 1, 2), (12, 4, 7), (8, 2, 16)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_multi_shapes(Hq, Hkv, T, d):
    q, kc, vc = _inputs(LENS, Hq, Hkv, T, 4100, d, 9000 + 10 * Hq + T)
    o, lse = _run(q, kc, vc, LENS, 1 / math.sqrt(d))
    ro, rl = oa.decode_multi(q, kc, vc, LENS, scale=1 / math.sqrt(d), dtype="bf16")
    _check_rows(o, lse, ro, rl, f"decode_multi Hq={Hq} Hkv={Hkv} T={T} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_multi_rope(d):
    q, kc, vc = _inputs(LENS, 16, 4, 4, 4100, d, 9400 + d)
    o, lse = _run(q, kc, vc, LENS, 1 / math.sqrt(d), rope_base=10000.0)
    ro, rl = oa.decode_multi(q, kc, vc, LENS, scale=1 / math.sqrt(d), rope_base=10000.0, dtype="bf16")
    _check_rows(o, lse, ro, rl, f"decode_multi rope d={d}")


def test_decode_multi_t1_equals_decode():
    import torch
    q, kc, vc = _inputs(LENS, 32, 8, 1, 4100, 128, 9500)
    a = _run(q, kc, vc, LENS, 0.0884)
    o, lse = esd.decode(dev(q[:, :, 0]), dev(kc), dev(vc), dev(LENS), scale=0.0884)
    torch.cuda.synchronize()
    assert np.array_equal(a[0][:, :, 0], host(o)) and np.array_equal(a[1][:, :, 0], host(lse))


def test_decode_multi_matches_prefill_rows():
    """One sequence with n cache rows and T new tokens equals the last T rows of
    causal attention over the n rows (bottom-right alignment)."""
    import torch
    n, T = 777, 6
    lens = np.array([n], dtype=np.int32)
    q, kc, vc = _inputs(lens, 8, 2, T, n, 128, 9600)
    o, lse = _run(q, kc, vc, lens, 0.0884)
    of, lf = esd.fwd(dev(q), dev(kc), dev(vc), causal=True, scale=0.0884)
    torch.cuda.synchronize()
    assert np.max(np.abs(o - host(of))) < 2e-2 and np.max(np.abs(lse - host(lf))) < 2e-3


def test_decode_multi_speculative_b32_shape():
    """The GQA decode batch (B=32, Hq=32, Hkv=8, d=128, lengths 1024..32768)
    verifying 4 drafted tokens per sequence: 16 queries per KV head, one pass."""
    w = W.WORKLOADS["decode_b32"]
    lens = W.decode_lens(w)
    _, kc, vc = W.decode_inputs(w, lens)
    q = W.normal((w.B, w.Hq, 4, w.d), 9700, 1.0, "bf16")
    say(f"decode_b32 shape with T=4: lens sum {lens.sum()}")
    o, lse = _run(q, kc, vc, lens, w.scale)
    ro, rl = oa.decode_multi(q, kc, vc, lens, scale=w.scale, dtype="bf16")
    _check_rows(o, lse, ro, rl, "decode_multi decode_b32 T=4")
