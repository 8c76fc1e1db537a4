"""GPU parity of paged-cache decode (attn_decode_paged) against the oracle.

Token p of sequence b lives in pool block table[b][p // block_size] at row
p % block_size ("Attention mechanisms: from alignment to efficient long
context", section 20).  The pools hold NaN in every row no sequence owns (spare
blocks, the tail of each last block) and the tables hold -1 past each
sequence's blocks, so a read of anything outside the sequence would show.
Tolerances as for contiguous decode (bf16: max|dO| <= 1e-2, max|dlse| <= 1e-3).
Paged and contiguous decode of the same rows are compared with each other too.
They split the cache into chunks of 1024 and 2048 keys, so each wave's reference
max, and with it the bf16 rounding of the weights, differs. The two therefore
agree to max|dO| <= 1e-3 (bf16 weight rounding) and max|dlse| <= 2e-5 (fp32 sums).
A key row read from the wrong place moves lse by about 1 / length, far more.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, dev, host, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")

LENS = np.array([0, 1, 2, 15, 16, 17, 31, 33, 127, 1023, 1024, 1025, 1040, 2047, 2048, 2049, 2100,
                 3000, 4112],
                dtype=np.int32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _run(q, kp, vp, table, lens, scale, rope_base=0.0):
    import torch
    o, lse = esd.decode_paged(dev(q), dev(kp), dev(vp), dev(table), dev(lens), scale=scale,
                              rope_base=rope_base)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _check_rows(o, lse, ro, rl, what):
    dead = np.isneginf(rl)
    assert np.array_equal(np.isneginf(lse), dead), what
    assert np.all(o[dead] == 0), what
    live = ~dead
    check(o[live], lse[live], ro[live], rl[live], "bf16", what)


@pytest.mark.parametrize("bs", [16, 32, 64, 256])
@pytest.mark.parametrize("Hq,Hkv,T", [(32, 8, 1), (32, 8, 4), (8, 8, 2), (16, 2, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_paged_shapes(bs, Hq, Hkv, T, d):
    w = W.WORKLOADS["decode_b32"]
    q, kp, vp, table = W.paged_inputs(w, LENS, block_size=bs, T=T, Hq=Hq, Hkv=Hkv, d=d,
                                      seed_base=9800 + bs + Hq + T + d)
    scale = 1 / math.sqrt(d)
    o, lse = _run(q, kp, vp, table, LENS, scale)
    ro, rl = oa.decode_paged(q, kp, vp, table, LENS, block_size=bs, scale=scale, dtype="bf16")
    _check_rows(o, lse, ro, rl, f"paged bs={bs} Hq={Hq} Hkv={Hkv} T={T} d={d}")


LENS_LONG = np.array([0, 1, 1023, 1024, 1025, 2048, 4095, 4096, 4097, 5000, 8192, 9001],
                     dtype=np.int32)


@pytest.mark.parametrize("bs", [512, 1024, 2048, 4096])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_paged_large_blocks(bs, d):
    """Blocks as long as a split workgroup's 1024-key chunk, or longer (up to the
    largest supported size): several chunks read one block, and a block's tail
    past the sequence length holds NaN that must never be read."""
    w = W.WORKLOADS["decode_b32"]
    q, kp, vp, table = W.paged_inputs(w, LENS_LONG, block_size=bs, T=2, Hq=16, Hkv=4, d=d,
                                      seed_base=9900 + bs + d)
    scale = 1 / math.sqrt(d)
    o, lse = _run(q, kp, vp, table, LENS_LONG, scale)
    ro, rl = oa.decode_paged(q, kp, vp, table, LENS_LONG, block_size=bs, scale=scale,
                             dtype="bf16")
    _check_rows(o, lse, ro, rl, f"paged bs={bs} d={d}")


@pytest.mark.parametrize("bs", [16, 128])
def test_decode_paged_equals_contiguous(bs):
    """The same rows laid out contiguously give the same outputs (to the rounding
    of the bf16 weights; lse to fp32 rounding)."""
    import torch
    w = W.WORKLOADS["decode_b32"]
    q, kp, vp, table = W.paged_inputs(w, LENS, block_size=bs, T=3, Hq=32, Hkv=8, d=128,
                                      seed_base=9900 + bs)
    o, lse = _run(q, kp, vp, table, LENS, 0.0884, rope_base=10000.0)
    max_len = int(LENS.max())
    kc = np.full((len(LENS), 8, max_len, 128), W.BF16_NAN_BITS, dtype=np.uint16)
    vc = kc.copy()
    for b, n in enumerate(LENS):
        pos = np.arange(n)
        kc[b, :, :n] = kp[table[b, pos // bs], :, pos % bs].transpose(1, 0, 2)
        vc[b, :, :n] = vp[table[b, pos // bs], :, pos % bs].transpose(1, 0, 2)
    oc, lc = esd.decode_multi(dev(q), dev(kc), dev(vc), dev(LENS), scale=0.0884, rope_base=10000.0)
    torch.cuda.synchronize()
    oc, lc = host(oc), host(lc)
    dead = np.isneginf(lc)
    assert np.array_equal(np.isneginf(lse), dead)
    assert np.all(o[dead] == 0) and np.all(oc[dead] == 0)
    do = float(np.max(np.abs(o[~dead].astype(np.float64) - oc[~dead])))
    dl = float(np.max(np.abs(lse[~dead].astype(np.float64) - lc[~dead])))
    say(f"paged bs={bs} vs contiguous: max|dO| = {do:.3e} (tol 1e-3), max|dlse| = {dl:.3e} (tol 2e-5)")
    assert do <= 1e-3 and dl <= 2e-5


def test_decode_paged_rope():
    w = W.WORKLOADS["decode_b32"]
    q, kp, vp, table = W.paged_inputs(w, LENS, block_size=16, T=2, Hq=16, Hkv=4, d=128,
                                      seed_base=9950)
    o, lse = _run(q, kp, vp, table, LENS, 0.0884, rope_base=10000.0)
    ro, rl = oa.decode_paged(q, kp, vp, table, LENS, block_size=16, scale=0.0884,
                             rope_base=10000.0, dtype="bf16")
    _check_rows(o, lse, ro, rl, "paged rope")


def test_decode_paged_b32_shape():
    """The GQA decode batch (B=32, Hq=32, Hkv=8, d=128, lengths 1024..32768) in
    16-token blocks scattered over the pool."""
    w = W.WORKLOADS["decode_b32"]
    lens = W.decode_lens(w)
    q, kp, vp, table = W.paged_inputs(w, lens, block_size=16)
    say(f"decode_b32 paged: {kp.shape[0]} blocks of 16, lens sum {lens.sum()}")
    o, lse = _run(q, kp, vp, table, lens, w.scale)
    ro, rl = oa.decode_paged(q, kp, vp, table, lens, block_size=16, scale=w.scale, dtype="bf16")
    _check_rows(o, lse, ro, rl, "paged decode_b32")
