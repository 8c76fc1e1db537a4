"""GPU parity at the edges of the shape space the kernels split into
workgroups: very large query-head groups (MQA with 128 query heads on one KV
head, so a group spans many workgroups and the dK/dV kernel visits 128 heads
per tile) and very many tiny sequences (thousands of (batch, head) units of a
few rows).  Against the oracle at the usual tolerances."""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, dev, host, say
from test_gpu_backward import _grad_check, _run

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def test_mqa_128_query_heads_forward_and_backward():
    """B=1, Hq=128, Hkv=1, N=200, d=128, causal, RoPE 1e4."""
    import torch
    B, Hq, Hkv, N, d = 1, 128, 1, 200, 128
    scale = 1 / math.sqrt(d)
    q = W.normal((B, Hq, N, d), 18001, 1.0, "bf16")
    k = W.normal((B, Hkv, N, d), 18002, 1.0, "bf16")
    v = W.normal((B, Hkv, N, d), 18003, 1.0, "bf16")
    do = W.normal((B, Hq, N, d), 18004, 1.0, "f32")
    say(f"MQA with {Hq} query heads, N={N}, d={d}")
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=True, scale=scale, rope_base=1e4)
    torch.cuda.synchronize()
    ro, rl = oa.attention(q, k, v, causal=True, scale=scale, rope_base=1e4, dtype="bf16")
    check(host(o), host(lse), ro, rl, "bf16", f"MQA {Hq} heads forward")
    got = _run(q, k, v, do, True, scale, 1e4)
    ref = oa.attention_bwd(q, k, v, do, causal=True, scale=scale, rope_base=1e4, dtype="bf16")
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        _grad_check(a, r, f"MQA {Hq} heads {name}")


@pytest.mark.parametrize("causal,Nq,Nk", [(True, 5, 5), (False, 3, 7)])
def test_many_tiny_sequences_forward(causal, Nq, Nk):
    """B=2048, Hq=4, Hkv=2, d=64: 4096 (batch, KV head) units of a few rows."""
    import torch
    B, Hq, Hkv, d = 2048, 4, 2, 64
    scale = 0.125
    q = W.normal((B, Hq, Nq, d), 18101, 1.0, "bf16")
    k = W.normal((B, Hkv, Nk, d), 18102, 1.0, "bf16")
    v = W.normal((B, Hkv, Nk, d), 18103, 1.0, "bf16")
    say(f"{B} tiny sequences, Nq={Nq} Nk={Nk} causal={causal}")
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oa.attention(q, k, v, causal=causal, scale=scale, dtype="bf16")
    check(host(o), host(lse), ro, rl, "bf16", f"{B} sequences forward")


def test_many_short_sequences_decode():
    """B=1024 sequences of 0-300 cached keys, Hq=8 on one KV head, d=128."""
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.random.default_rng(18201).integers(0, 301, 1024).astype(np.int32)
    q, kc, vc = W.decode_inputs(w, lens, Hq=8, Hkv=1, max_len=300, d=128, seed_base=18200)
    say("decode: 1024 sequences of 0-300 keys")
    o, lse = esd.decode(dev(q), dev(kc), dev(vc), dev(lens), scale=1 / math.sqrt(128))
    torch.cuda.synchronize()
    ro, rl = oa.decode(q, kc, vc, lens, scale=1 / math.sqrt(128))
    o, lse = host(o), host(lse)
    empty = lens == 0
    # a sequence with no key yields O = 0 and lse = -inf
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    check(o[~empty], lse[~empty], ro[~empty], rl[~empty], "bf16", "decode 1024 sequences")
