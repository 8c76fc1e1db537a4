"""The work the benchmark divides by: FLOPs per visible (query, key) pair and
the decode's algorithmic bytes, pinned to the figures stated for each workload
and to a brute-force count of the visible pairs.  CPU only."""

import numpy as np
import pytest

import bench
import workloads as W


@pytest.mark.parametrize("name,flops", [
    ("f32_n256", 16_777_216),               # 4 d N^2, non-causal, d = 64
    ("mha_d64_n2048", 34_376_515_584),      # 4 d (N (N + 1) / 2) B H
    ("gqa_rope_n8192", 1_099_645_845_504),  # ~1.09965e12
    ("gqa_rope_n32768", 17_592_722_915_328),  # ~1.75927e13
])
def test_workload_flops(name, flops):
    assert bench.fwd_flops(W.WORKLOADS[name]) == flops


def test_decode_batch_lengths_and_bytes():
    w = W.WORKLOADS["decode_b32"]
    lens = W.decode_lens(w)
    assert (int(lens.min()), int(lens.max()), int(lens.sum())) == (1349, 32575, 638284)
    # every valid K and V row once (bf16), plus q (bf16), o and lse (fp32), lens (int32)
    kv = 638284 * 8 * 128 * 2 * 2
    assert kv == 2_614_411_264
    assert bench.decode_bytes(w, lens) == kv + 32 * 32 * 128 * 2 + 32 * 32 * 128 * 4 + 32 * 32 * 4 + 32 * 4
    assert bench.decode_bytes(w, lens) == 2_615_201_920


def _brute(Nq, Nk, causal, window):
    qpos = np.arange(Nq)[:, None] + (Nk - Nq)
    kpos = np.arange(Nk)[None, :]
    vis = np.ones((Nq, Nk), bool)
    if causal:
        vis &= kpos <= qpos
    if window:
        vis &= kpos > qpos - window
    return int(vis.sum())


@pytest.mark.parametrize("Nq,Nk,causal,window", [
    (1, 1, True, 0), (7, 7, True, 0), (5, 9, True, 0), (64, 64, False, 0), (3, 11, False, 0),
    (100, 100, True, 1), (100, 100, True, 7), (37, 90, True, 16), (90, 90, True, 200),
])
def test_visible_pairs_brute_force(Nq, Nk, causal, window):
    assert bench.visible_pairs(Nq, Nk, causal, window) == _brute(Nq, Nk, causal, window)
