"""Out-of-range lengths and block-table entries in the decode calls.

The header defines them: sequence lengths are clamped to [0, max_len] (to
[0, max_blocks * block_size] for a paged cache), and the table entries of the
blocks a sequence uses are clamped into [0, num_blocks).  Each call with
out-of-range values must equal, bit for bit, the same call with the values
clamped by hand, and the contiguous case must match the oracle on the clamped
lengths."""

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


def _same(a, b):
    return np.array_equal(host(a), host(b), equal_nan=True)


def test_decode_lengths_are_clamped():
    import torch
    w = W.WORKLOADS["decode_b32"]
    max_len, d = 300, 64
    raw = np.array([-5, 0, 1, 137, max_len, max_len + 100, 2**31 - 1, -2**31], dtype=np.int32)
    clamped = np.clip(raw, 0, max_len).astype(np.int32)
    q, kc, vc = W.decode_inputs(w, clamped, Hq=8, Hkv=2, max_len=max_len, d=d, seed_base=18300)
    say(f"decode with lengths {raw.tolist()}")
    dq, dkc, dvc = dev(q), dev(kc), dev(vc)
    o1, l1 = esd.decode(dq, dkc, dvc, dev(raw), scale=0.125)
    o2, l2 = esd.decode(dq, dkc, dvc, dev(clamped), scale=0.125)
    torch.cuda.synchronize()
    assert _same(o1, o2) and _same(l1, l2)
    ro, rl = oa.decode(q, kc, vc, clamped, scale=0.125)
    keep = clamped > 0
    check(host(o1)[keep], host(l1)[keep], ro[keep], rl[keep], "bf16", "decode, clamped lengths")
    assert np.all(host(o1)[~keep] == 0) and np.all(np.isneginf(host(l1)[~keep]))
    # several new tokens: their positions follow the clamped length too
    T = 2
    qm = W.normal((len(raw), 8, T, d), 18310, 1.0, "bf16")
    m1, n1 = esd.decode_multi(dev(qm), dkc, dvc, dev(raw), scale=0.125)
    m2, n2 = esd.decode_multi(dev(qm), dkc, dvc, dev(clamped), scale=0.125)
    torch.cuda.synchronize()
    assert _same(m1, m2) and _same(n1, n2)


def test_paged_table_entries_and_lengths_are_clamped():
    import torch
    w = W.WORKLOADS["decode_b32"]
    bs, d = 16, 64
    lens = np.array([40, 17, 0, 64], dtype=np.int32)
    q, kp, vp, table = W.paged_inputs(w, lens, block_size=bs, T=1, Hq=8, Hkv=2, d=d,
                                      seed_base=18400)
    num_blocks, max_blocks = kp.shape[0], table.shape[1]
    raw_t, clamp_t = table.copy(), table.copy()
    raw_t[1, 0], clamp_t[1, 0] = -7, 0                            # used blocks, out of range
    raw_t[1, 1], clamp_t[1, 1] = num_blocks + 3, num_blocks - 1
    raw_l, clamp_l = lens.copy(), lens.copy()
    raw_l[2], clamp_l[2] = -9, 0
    raw_l[3], clamp_l[3] = max_blocks * bs + 50, max_blocks * bs
    say(f"paged decode: table entries -7 and {num_blocks + 3} of {num_blocks} blocks, "
        f"lengths {raw_l.tolist()}")
    dq, dkp, dvp = dev(q), dev(kp), dev(vp)
    o1, l1 = esd.decode_paged(dq, dkp, dvp, dev(raw_t), dev(raw_l), scale=1 / math.sqrt(d))
    o2, l2 = esd.decode_paged(dq, dkp, dvp, dev(clamp_t), dev(clamp_l), scale=1 / math.sqrt(d))
    torch.cuda.synchronize()
    assert _same(o1, o2) and _same(l1, l2)
