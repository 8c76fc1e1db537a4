"""GPU parity of chunked prefill over a cache (attn_prefill_cached) and of the
optional bf16 O of the chunked-prefill and multi-token decode calls.

attn_prefill_cached: Nq new tokens are the last Nq rows of a cache of Nk rows
whose keys are stored already rotated; query i sits at Nk - Nq + i and sees
keys 0 .. Nk - Nq + i ("coding-interview attention from scratch", 八 question
5).  That is the oracle's multi-token decode with every sequence holding Nk
rows and T = Nq, which is what it is compared with.  Run on keys rotated by
attn_rope_apply it must equal attn_fwd with RoPE bit for bit: it is the same
attention kernel without the rotation pass of K.

bf16 O: the GPU rounds its fp32 O to the nearest bf16; the oracle's O is
rounded fp64 -> fp32 -> bf16; compared within the bf16 tolerance plus one bf16
spacing (the two sides round values up to 1e-2 apart).
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, check_bf16_o, dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype, sigma=1.0):
    q = W.normal((B, Hq, Nq, d), seed + 1, sigma, dtype)
    k = W.normal((B, Hkv, Nk, d), seed + 2, sigma, dtype)
    v = W.normal((B, Hkv, Nk, d), seed + 3, 1.0, dtype)
    return q, k, v


def _ref(q, k, v, scale, rope_base, dtype):
    B, Nk = q.shape[0], k.shape[2]
    return oa.decode_multi(q, k, v, np.full(B, Nk), scale=scale, rope_base=rope_base, dtype=dtype)


CASES = [
    # dtype, d, Hq, Hkv, Nq, Nk, rope_base
    ("bf16", 128, 8, 2, 1, 1, 0.0),
    ("bf16", 128, 8, 2, 7, 300, 10000.0),
    ("bf16", 128, 8, 2, 129, 129, 10000.0),
    ("bf16", 128, 32, 8, 200, 1000, 500000.0),
    ("bf16", 64, 4, 4, 65, 130, 10000.0),
    ("bf16", 64, 16, 1, 97, 200, 0.0),
    ("f32", 128, 4, 2, 33, 100, 10000.0),
    ("f32", 64, 4, 1, 65, 65, 0.0),
]


@pytest.mark.parametrize("dtype,d,Hq,Hkv,Nq,Nk,base", CASES)
def test_prefill_cached(dtype, d, Hq, Hkv, Nq, Nk, base):
    import torch
    q, k, v = _inputs(15000 + Nq + Nk + d, 2, Hq, Hkv, Nq, Nk, d, dtype, sigma=2.0)
    # the cache holds the keys rotated, as a decoder would have stored them
    kr = oa.rope(W.as_f64(k, dtype), np.arange(Nk), base, dtype) if base else W.as_f64(k, dtype)
    kr = (W.f32_to_bf16_bits(kr.astype(np.float32)) if dtype == "bf16" else kr.astype(np.float32))
    scale = 1.0 / math.sqrt(d)
    o, lse = esd.prefill_cached(dev(q), dev(kr), dev(v), scale=scale, rope_base=base)
    torch.cuda.synchronize()
    ro, rl = _ref(q, kr, v, scale, base, dtype)
    check(host(o), host(lse), ro, rl, dtype, f"prefill_cached {dtype} d={d} Hq={Hq} Hkv={Hkv} "
          f"Nq={Nq} Nk={Nk} base={base}")


@pytest.mark.parametrize("d,Nq,Nk", [(128, 8192, 8192), (128, 333, 1000), (64, 100, 100)])
def test_prefill_cached_equals_fwd_on_rotated_keys(d, Nq, Nk):
    """attn_rope_apply(k) then attn_prefill_cached == attn_fwd(causal, RoPE), bit
    for bit, including the causal GQA N=8192 shape the benchmark times."""
    import torch
    B, Hq, Hkv = (2, 32, 8) if Nq == 8192 else (1, 8, 2)
    q, k, v = _inputs(15500 + Nq + d, B, Hq, Hkv, Nq, Nk, d, "bf16")
    tq, tk, tv = dev(q), dev(k), dev(v)
    o1, l1 = esd.fwd(tq, tk, tv, causal=True, scale=1 / math.sqrt(d), rope_base=10000.0)
    kr = esd.rope_apply(tk, 10000.0, 0)
    o2, l2 = esd.prefill_cached(tq, kr, tv, scale=1 / math.sqrt(d), rope_base=10000.0)
    torch.cuda.synchronize()
    say(f"prefill_cached vs fwd B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d}")
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype,d,Nq,Nk,base", [("bf16", 128, 200, 700, 10000.0),
                                                ("bf16", 64, 65, 65, 0.0),
                                                ("f32", 128, 40, 90, 10000.0)])
def test_prefill_cached_bf16_out(dtype, d, Nq, Nk, base):
    import torch
    q, k, v = _inputs(15800 + Nq + d, 1, 8, 2, Nq, Nk, d, dtype, sigma=2.0)
    kr = oa.rope(W.as_f64(k, dtype), np.arange(Nk), base, dtype) if base else W.as_f64(k, dtype)
    kr = (W.f32_to_bf16_bits(kr.astype(np.float32)) if dtype == "bf16" else kr.astype(np.float32))
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = dev(q), dev(kr), dev(v)
    o, lse = esd.prefill_cached(tq, tk, tv, scale=scale, rope_base=base, out_dtype=torch.bfloat16)
    o32, l32 = esd.prefill_cached(tq, tk, tv, scale=scale, rope_base=base)
    torch.cuda.synchronize()
    assert o.dtype == torch.bfloat16
    # the bf16 O is the fp32 O rounded to nearest even (torch's own conversion)
    assert torch.equal(o, o32.to(torch.bfloat16)) and torch.equal(lse, l32)
    ro, rl = _ref(q, kr, v, scale, base, dtype)
    check_bf16_o(host(o.float()), host(lse), ro, rl, f"prefill_cached bf16 O {dtype} d={d}")


LENS = np.array([0, 1, 3, 33, 1023, 2049, 4097], dtype=np.int32)


@pytest.mark.parametrize("T,d,base", [(1, 128, 0.0), (4, 128, 10000.0), (3, 64, 0.0)])
def test_decode_multi_bf16_out(T, d, base):
    import torch
    w = W.WORKLOADS["decode_b32"]
    _, kc, vc = W.decode_inputs(w, LENS, Hq=8, Hkv=2, max_len=4100, d=d, seed_base=16000 + T)
    q = W.normal((len(LENS), 8, T, d), 16007 + T, 1.0, "bf16")
    tq, tk, tv, tl = dev(q), dev(kc), dev(vc), dev(LENS)
    o, lse = esd.decode_multi(tq, tk, tv, tl, scale=1 / math.sqrt(d), rope_base=base,
                              out_dtype=torch.bfloat16)
    o32, l32 = esd.decode_multi(tq, tk, tv, tl, scale=1 / math.sqrt(d), rope_base=base)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(torch.bfloat16)) and torch.equal(lse, l32)
    ro, rl = oa.decode_multi(q, kc, vc, LENS, scale=1 / math.sqrt(d), rope_base=base, dtype="bf16")
    dead = np.isneginf(rl)
    og = host(o.float())
    assert np.all(og[dead] == 0) and np.array_equal(np.isneginf(host(lse)), dead)
    check_bf16_o(og[~dead], host(lse)[~dead], ro[~dead], rl[~dead], f"decode_multi bf16 O T={T} d={d}")


def test_decode_paged_bf16_out():
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.array([5, 300, 2100], dtype=np.int32)
    q, kp, vp, table = W.paged_inputs(w, lens, block_size=16, T=2, Hq=8, Hkv=2, seed_base=16100)
    args = (dev(q), dev(kp), dev(vp), dev(table), dev(lens))
    o, lse = esd.decode_paged(*args, scale=w.scale, out_dtype=torch.bfloat16)
    o32, l32 = esd.decode_paged(*args, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(torch.bfloat16)) and torch.equal(lse, l32)
    ro, rl = oa.decode_paged(q, kp, vp, table, lens, block_size=16, scale=w.scale, dtype="bf16")
    check_bf16_o(host(o.float()), host(lse), ro, rl, "decode_paged bf16 O")
