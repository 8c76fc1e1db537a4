"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances: bf16 inputs max|dO| <= 1e-2 and max|dlse| <= 1e-3; fp32 inputs
1e-4 on both.  Small shapes are compared element by element; the full-size
workloads in the launch configuration the benchmark times: every output of the
fp32 single-head case, the MHA causal case, the causal GQA N=8192 case and
decode; all 64 heads of the N=32768 case at the edges of sampled row blocks.
"""

import math

import numpy as np
import pytest

import oracle.dense as oa
import workloads as W
from gpu_util import check, dev, host, max_err, say

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _run_fwd(q, k, v, dtype, causal, scale, rope_base):
    import torch
    o, lse = esd.fwd(dev(q), dev(k), dev(v), causal=causal, scale=scale, rope_base=rope_base)
    torch.cuda.synchronize()
    return host(o), host(lse)


def _small_inputs(seed, B, Hq, Hkv, Nq, Nk, d, dtype, sigma=1.0):
    q = W.normal((B, Hq, Nq, d), seed + 1, sigma, dtype)
    k = W.normal((B, Hkv, Nk, d), seed + 2, sigma, dtype)
    v = W.normal((B, Hkv, Nk, d), seed + 3, 1.0, dtype)
    return q, k, v


SMALL = []
for dtype in ("bf16", "f32"):
    for d in (64, 128):
        for (Nq, Nk) in [(1, 1), (7, 7), (63, 63), (65, 65), (129, 129), (1, 129), (7, 65),
                         (65, 129), (129, 300)]:
            for causal in (False, True):
                SMALL.append((dtype, d, Nq, Nk, causal))


@pytest.mark.parametrize("dtype,d,Nq,Nk,causal", SMALL)
def test_small_ragged(dtype, d, Nq, Nk, causal):
    """Ragged tails of tiles and rows, causal with Nq <= Nk (bottom-right)."""
    B, Hq, Hkv = 1, 4, 2
    q, k, v = _small_inputs(7000 + Nq * 3 + Nk, B, Hq, Hkv, Nq, Nk, d, dtype)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(q, k, v, dtype, causal, scale, 0.0)
    ro, rl = oa.attention(q, k, v, causal=causal, scale=scale, dtype=dtype)
    check(o, lse, ro, rl, dtype, f"{dtype} d={d} Nq={Nq} Nk={Nk} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(300, 129), (129, 7), (65, 1)])
def test_more_queries_than_keys_unmasked(dtype, d, Nq, Nk):
    """No mask and more queries than keys (allowed without a mask or RoPE):
    every query sees all Nk keys, including a single key."""
    q, k, v = _small_inputs(12100 + Nq + Nk + d, 1, 4, 2, Nq, Nk, d, dtype)
    o, lse = _run_fwd(q, k, v, dtype, False, 1 / math.sqrt(d), 0.0)
    ro, rl = oa.attention(q, k, v, causal=False, scale=1 / math.sqrt(d), dtype=dtype)
    check(o, lse, ro, rl, dtype, f"unmasked Nq={Nq} > Nk={Nk} d={d} {dtype}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (16, 2), (12, 4), (6, 2), (3, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_head_sharing(Hq, Hkv, dtype):
    """MHA, GQA (groups of 2..8, also non-power-of-two groups) and MQA."""
    q, k, v = _small_inputs(7100 + Hq * 10 + Hkv, 2, Hq, Hkv, 100, 100, 128, dtype)
    o, lse = _run_fwd(q, k, v, dtype, True, 0.0884, 0.0)
    ro, rl = oa.attention(q, k, v, causal=True, scale=0.0884, dtype=dtype)
    check(o, lse, ro, rl, dtype, f"Hq={Hq} Hkv={Hkv} {dtype}")


@pytest.mark.parametrize("Hq,Hkv", [(10, 2), (12, 2), (7, 1), (24, 2), (32, 2)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_group_sizes_split_over_workgroups(Hq, Hkv, d, causal):
    """Group sizes 5, 6, 7, 12 and 16: the heads of one KV head are spread over
    one or several workgroups (a common divisor of the group size and the wave
    count per workgroup), with a ragged row tail."""
    q, k, v = _small_inputs(7150 + Hq * 10 + Hkv + d, 1, Hq, Hkv, 77, 140, d, "bf16")
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(q, k, v, "bf16", causal, scale, 0.0)
    ro, rl = oa.attention(q, k, v, causal=causal, scale=scale, dtype="bf16")
    check(o, lse, ro, rl, "bf16", f"Hq={Hq} Hkv={Hkv} d={d} causal={causal}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("base", [10000.0, 500000.0, 10.0])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_attention_small(dtype, base, d):
    q, k, v = _small_inputs(7200 + d, 1, 8, 2, 150, 200, d, dtype, sigma=2.0)
    scale = 1.0 / math.sqrt(d)
    o, lse = _run_fwd(q, k, v, dtype, True, scale, base)
    ro, rl = oa.attention(q, k, v, causal=True, scale=scale, rope_base=base, dtype=dtype)
    check(o, lse, ro, rl, dtype, f"rope base={base} d={d} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("base,N,off", [(10000.0, 300, 0), (500000.0, 4096, 28672), (10.0, 64, 5),
                                         (10000.0, 1000, (1 << 22) - 1000)])
def test_rope_apply_bit_exact(dtype, base, N, off):
    """The device rotation rounds to exactly the oracle's values, up to the
    largest position any call accepts (2^22 - 1)."""
    d = 128
    x = W.normal((2, 3, N, d), 7300 + N, 4.0, dtype)
    got = host(esd.rope_apply(dev(x), base, pos_offset=off))
    xf = W.as_f64(x, dtype)
    ref = oa.rope(xf.reshape(-1, N, d), np.arange(N) + off, base, dtype).reshape(xf.shape)
    g = W.as_f64(got, dtype)
    bad = int(np.sum(g != ref))
    say(f"rope_apply {dtype} base={base} N={N} off={off}: {bad} mismatching elements")
    assert bad == 0


def test_causal_row0_and_uniform_scores():
    """Query 0 of causal attention returns V[0] exactly; Q = 0 returns the mean of
    the visible V rows and lse = ln(count)."""
    q, k, v = _small_inputs(7400, 1, 4, 2, 200, 200, 128, "bf16")
    o, lse = _run_fwd(q, k, v, "bf16", True, 0.0884, 10000.0)
    vf = W.as_f64(v, "bf16")
    for h in range(4):
        assert np.array_equal(o[0, h, 0].astype(np.float64), vf[0, h // 2, 0])
    qz = np.zeros_like(q)
    o, lse = _run_fwd(qz, k, v, "bf16", True, 0.0884, 0.0)
    for i in (0, 1, 100, 199):
        assert max_err(o[0, 0, i], vf[0, 0, :i + 1].mean(0)) < 1e-2
        assert abs(lse[0, 0, i] - math.log(i + 1)) < 1e-5


def test_deterministic():
    q, k, v = _small_inputs(7500, 2, 8, 2, 333, 333, 128, "bf16")
    a = _run_fwd(q, k, v, "bf16", True, 0.0884, 10000.0)
    b = _run_fwd(q, k, v, "bf16", True, 0.0884, 10000.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------- full sizes
def test_f32_n256_full():
    w = W.WORKLOADS["f32_n256"]
    q, k, v = W.fwd_inputs(w)
    say("f32_n256: fp32 non-causal B=1 H=1 N=256 d=64")
    o, lse = _run_fwd(q, k, v, "f32", False, w.scale, 0.0)
    ro, rl = oa.attention(q, k, v, causal=False, scale=w.scale, dtype="f32")
    check(o, lse, ro, rl, "f32", "f32_n256 all outputs")


def test_mha_d64_n2048_full():
    w = W.WORKLOADS["mha_d64_n2048"]
    q, k, v = W.fwd_inputs(w)
    say("mha_d64_n2048: bf16 causal MHA B=4 H=16 N=2048 d=64")
    o, lse = _run_fwd(q, k, v, "bf16", True, w.scale, 0.0)
    ro, rl = oa.attention(q, k, v, causal=True, scale=w.scale, dtype="bf16")
    check(o, lse, ro, rl, "bf16", "mha_d64_n2048 all outputs")


def test_gqa_rope_n8192_every_row():
    """Causal GQA + RoPE 1e4, B=2 Hq=32 Hkv=8 N=8192 d=128, in the launch
    configuration the benchmark times: every (batch, head) and every row
    against the oracle."""
    w = W.WORKLOADS["gqa_rope_n8192"]
    q, k, v = W.fwd_inputs(w)
    say(f"{w.name}: {w.note}")
    o, lse = _run_fwd(q, k, v, w.dtype, w.causal, w.scale, w.rope_base)
    rows = np.arange(w.Nq)
    kc = {}
    eo = el = 0.0
    for b in range(w.B):
        for h in range(w.Hq):
            ro, rl = oa.attention_rows(q, k, v, b, h, rows, causal=True, scale=w.scale,
                                       rope_base=w.rope_base, dtype=w.dtype, _kcache=kc)
            assert np.all(np.isfinite(o[b, h])) and np.all(np.isfinite(lse[b, h]))
            eo = max(eo, max_err(o[b, h], ro))
            el = max(el, max_err(lse[b, h], rl))
        say(f"{w.name}: batch {b} done, max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= 1e-2 and el <= 1e-3, (eo, el)


def _block_edge_rows(N, rows_per_block, rng, n_blocks, n_random):
    """Rows at both edges of sampled workgroup row blocks and of the 32-row
    wave blocks inside them, plus random rows; the first and last blocks are
    always sampled."""
    nrb = (N + rows_per_block - 1) // rows_per_block
    blocks = np.unique(np.concatenate([[0, 1, nrb // 2, nrb - 2, nrb - 1],
                                       rng.integers(0, nrb, n_blocks)]))
    rows = []
    for blk in blocks:
        r0 = blk * rows_per_block
        for off in range(0, rows_per_block, 32):
            rows += [r0 + off, r0 + off + 31]
    rows = np.asarray(rows)
    rows = np.concatenate([rows[rows < N], rng.integers(0, N, n_random)])
    return np.unique(rows)


def test_gqa_rope_n32768_all_heads_block_edges():
    """Long-context GQA + RoPE 5e5, B=1 Hq=64 Hkv=8 N=32768 d=128, Q,K ~ N(0,16):
    all 64 heads, each on at least 128 rows at both edges of 64-row workgroup
    blocks (the 8 query heads of a KV head share its tiles in one workgroup,
    one wave of 64 rows per head) and of the two 32-row blocks of each wave,
    at blocks sampled per head."""
    w = W.WORKLOADS["gqa_rope_n32768"]
    q, k, v = W.fwd_inputs(w)
    say(f"{w.name}: {w.note}")
    o, lse = _run_fwd(q, k, v, w.dtype, w.causal, w.scale, w.rope_base)
    rng = np.random.default_rng(5)
    kc = {}
    eo = el = 0.0
    for h in range(w.Hq):
        rows = _block_edge_rows(w.Nq, 64, rng, 32, 12)
        assert len(rows) >= 128, len(rows)
        ro, rl = oa.attention_rows(q, k, v, 0, h, rows, causal=True, scale=w.scale,
                                   rope_base=w.rope_base, dtype=w.dtype, _kcache=kc)
        assert np.all(np.isfinite(o[0, h, rows])) and np.all(np.isfinite(lse[0, h, rows]))
        eo = max(eo, max_err(o[0, h, rows], ro))
        el = max(el, max_err(lse[0, h, rows], rl))
    say(f"{w.name}: 64 heads, max|dO|={eo:.3e} max|dlse|={el:.3e}")
    assert eo <= 1e-2 and el <= 1e-3, (eo, el)


def test_decode_b32_full():
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = W.decode_lens(w)
    q, kc, vc = W.decode_inputs(w, lens)
    say(f"decode_b32: {w.note}; lens min {lens.min()} max {lens.max()} sum {lens.sum()}")
    o, lse = esd.decode(dev(q), dev(kc), dev(vc), dev(lens), scale=w.scale)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    ro, rl = oa.decode(q, kc, vc, lens, scale=w.scale)
    check(o, lse, ro, rl, "bf16", "decode_b32 all outputs")


# ----------------------------------------------------------------- decode edges
@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (32, 8), (16, 2), (32, 1), (12, 4), (64, 2)])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_shapes(Hq, Hkv, d):
    """Lengths 0, 1, batch / wave / chunk edges (32, 256, 2048 keys), several
    chunks, and a NaN-poisoned tail past each length."""
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.array([0, 1, 31, 33, 127, 129, 1023, 1024, 1025, 2047, 2048, 2049, 3000, 4097],
                    dtype=np.int32)
    q, kc, vc = W.decode_inputs(w, lens, Hq=Hq, Hkv=Hkv, max_len=4100, d=d, seed_base=7600 + Hq)
    o, lse = esd.decode(dev(q), dev(kc), dev(vc), dev(lens), scale=1 / math.sqrt(d))
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    ro, rl = oa.decode(q, kc, vc, lens, scale=1 / math.sqrt(d))
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    check(o[1:], lse[1:], ro[1:], rl[1:], "bf16", f"decode Hq={Hq} Hkv={Hkv} d={d}")


def test_decode_matches_fwd_last_row():
    """Decode over n cached keys equals causal prefill's last row (same library)."""
    import torch
    n, d = 777, 128
    q, k, v = _small_inputs(7700, 1, 8, 2, n, n, d, "bf16")
    o_f, l_f = _run_fwd(q, k, v, "bf16", True, 1 / math.sqrt(d), 0.0)
    lens = np.array([n], dtype=np.int32)
    o_d, l_d = esd.decode(dev(np.ascontiguousarray(q[:, :, n - 1])), dev(k), dev(v), dev(lens),
                          scale=1 / math.sqrt(d))
    torch.cuda.synchronize()
    assert max_err(host(o_d), o_f[:, :, n - 1]) < 2e-3
    assert max_err(host(l_d), l_f[:, :, n - 1]) < 1e-4


def test_fwd_errors_raise():
    import torch
    q = torch.zeros((1, 3, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(esd.AttnError):
        esd.fwd(q, k, k, causal=True)
    q = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(esd.AttnError):
        esd.fwd(q, q, q, causal=True)


def test_decode_more_chunks_than_merge_slots():
    """A 2.2M-key sequence: 1075 partial states of 2048 keys, more than the 1024
    weights the merge kernel keeps in LDS, so the rest are recomputed."""
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.array([2_200_000, 5], dtype=np.int32)
    q, kc, vc = W.decode_inputs(w, lens, Hq=4, Hkv=1, max_len=2_200_000, d=64, seed_base=7900)
    say("decode: one sequence of 2.2M keys (1075 chunks)")
    o, lse = esd.decode(dev(q), dev(kc), dev(vc), dev(lens), scale=0.125)
    torch.cuda.synchronize()
    ro, rl = oa.decode(q, kc, vc, lens, scale=0.125)
    check(host(o), host(lse), ro, rl, "bf16", "decode 2.2M keys")
