"""attn_decode_noalloc (the decode entry point without a workspace, for
callers that cannot allocate) against attn_decode through the C ABI: two calls
in a row, the second smaller, each bit-identical to attn_decode on the same
inputs and within the bf16 tolerance of the fp64 oracle."""

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


def _one(lens, Hq, Hkv, max_len, d, seed_base, what):
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.asarray(lens, dtype=np.int32)
    q, kc, vc = W.decode_inputs(w, lens, Hq=Hq, Hkv=Hkv, max_len=max_len, d=d,
                                seed_base=seed_base)
    need = esd.decode_workspace_bytes(len(lens), Hq, Hkv, max_len, d)
    assert need <= esd.DECODE_NOALLOC_MAX_BYTES
    say(f"{what}: B={len(lens)} Hq={Hq} Hkv={Hkv} max_len={max_len} d={d} "
        f"(partial states {need} bytes)")
    tq, tk, tv, tl = dev(q), dev(kc), dev(vc), dev(lens)
    o_ref, l_ref = esd.decode(tq, tk, tv, tl, scale=1 / math.sqrt(d))
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    torch.cuda.synchronize()
    esd.decode_noalloc(tq, tk, tv, tl, scale=1 / math.sqrt(d), out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), what
    ro, rl = oa.decode(q, kc, vc, lens, scale=1 / math.sqrt(d))
    live = lens > 0
    check(host(o)[live], host(lse)[live], ro[live], rl[live], "bf16", what)
    assert np.all(host(o)[~live] == 0) and np.all(np.isneginf(host(lse)[~live]))


def test_noalloc_two_calls_second_smaller():
    w = W.WORKLOADS["decode_b32"]
    # first: the full decode batch (32 sequences, lengths 1349 .. 32575)
    _one(W.decode_lens(w), w.Hq, w.Hkv, w.max_len, w.d, 4000, "noalloc call 1 (decode batch)")
    # second: fewer sequences, shorter caches, other heads and head dim; the
    # array still holds the first call's partial states
    _one([0, 1, 300, 2049, 5000], 8, 2, 5000, 64, 14200, "noalloc call 2 (smaller)")
