"""GPU parity at the largest key length the forward accepts.

attn_fwd takes one head's K (and V) below 2 GiB at fp32 size, Nk * d * 4 <
2^31, and RoPE positions below 2^22: at d = 128 both allow at most Nk =
4194303 keys.  These cases put the buffer offsets of the kernels at that
limit, with a ragged number of queries (two 32-row blocks and three rows) at
the bottom-right end of the causal mask, against the oracle at the usual
tolerances.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import dev, host, max_err, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")

NK_MAX = (1 << 31) // (128 * 4) - 1  # 4194303


def test_nk_limit_values():
    # the largest Nk the host accepts at d = 128, and the RoPE position limit
    assert NK_MAX * 128 * 4 < (1 << 31) <= (NK_MAX + 1) * 128 * 4
    assert NK_MAX < (1 << 22)


def test_max_keys_bf16():
    """bf16, causal GQA (2 query heads on 1 KV head), 67 queries at positions
    Nk-67 .. Nk-1 against Nk = 4194303 keys, at the edges of the 32-row blocks
    of both heads.  (The top RoPE positions are covered bit for bit by the
    rotation test at offset 2^22 - 1000; rotating 4M keys in the fp64 oracle
    would take minutes.)"""
    import torch
    d, Nq, Nk = 128, 67, NK_MAX
    scale = 1 / math.sqrt(d)
    say(f"max keys bf16: B=1 Hq=2 Hkv=1 Nq={Nq} Nk={Nk} d={d} (generating inputs)")
    q = W.normal((1, 2, Nq, d), 17001, 1.0, "bf16")
    k = W.normal((1, 1, Nk, d), 17002, 1.0, "bf16")
    v = W.normal((1, 1, Nk, d), 17003, 1.0, "bf16")
    say("max keys bf16: attn_fwd")
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=True, scale=scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    torch.cuda.empty_cache()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    say("max keys bf16: oracle")
    eo = el = 0.0
    for h, rows in ((0, np.array([0, 1, 2, 31, 32, 33, 63, 64, 65, 66])), (1, np.array([0, 32, 66]))):
        ro, rl = oa.attention_rows(q, k, v, 0, h, rows, causal=True, scale=scale, dtype="bf16")
        eo = max(eo, max_err(o[0, h, rows], ro))
        el = max(el, max_err(lse[0, h, rows], rl))
    say(f"max keys bf16: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= 1e-2 and el <= 1e-3, (eo, el)


def test_max_keys_f32():
    """fp32, one head, no mask, 5 queries against Nk = 4194303 keys: K and V
    of the head take 2 GiB less 512 bytes each."""
    import torch
    d, Nq, Nk = 128, 5, NK_MAX
    scale = 1 / math.sqrt(d)
    say(f"max keys f32: B=1 H=1 Nq={Nq} Nk={Nk} d={d} (generating inputs)")
    q = W.normal((1, 1, Nq, d), 17101, 1.0, "f32")
    k = W.normal((1, 1, Nk, d), 17102, 1.0, "f32")
    v = W.normal((1, 1, Nk, d), 17103, 1.0, "f32")
    assert k.nbytes == (1 << 31) - 512
    say("max keys f32: attn_fwd")
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=False, scale=scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    torch.cuda.empty_cache()
    say("max keys f32: oracle")
    ro, rl = oa.attention_rows(q, k, v, 0, 0, np.arange(Nq), causal=False, scale=scale,
                               dtype="f32")
    eo, el = max_err(o[0, 0], ro), max_err(lse[0, 0], rl)
    say(f"max keys f32: max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= 1e-4 and el <= 1e-4, (eo, el)
