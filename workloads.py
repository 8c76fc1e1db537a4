"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the attention arithmetic.  Both the fp64 oracle (through the
tests) and the GPU path are fed from it, so the two sides see bit-identical
inputs.

Workloads (shapes follow the pages' own examples: n = 8192 with d = 128 and
32 query / 8 KV heads as in Llama-3-8B, 64 query / 8 KV heads as in
LLaMA-3-70B, a decode batch of 32 sequences):

* ``f32_n256`` single-head non-causal fp32, B=1 H=1 N=256 d=64
* ``mha_d64_n2048`` MHA causal prefill bf16, B=4 H=16 N=2048 d=64
* ``gqa_rope_n8192`` GQA causal prefill bf16 with RoPE base 10000, B=2 Hq=32 Hkv=8 N=8192 d=128
* ``decode_b32`` GQA decode bf16, B=32 Hq=32 Hkv=8 d=128, KV lengths ~ U[1024, 32768]
* ``gqa_rope_n32768`` long-context GQA causal prefill bf16 with RoPE base 500000,
  B=1 Hq=64 Hkv=8 N=32768 d=128, Q and K ~ N(0, 4^2)

Recipe: ``numpy.random.default_rng(seed).standard_normal(shape, float32) * sigma``,
rounded to bf16 with round-to-nearest-even (fp32 workloads stay fp32).
Seeds are ``seed_base + t`` with t = 1, 2, 3 for Q, K, V (seed_base 1000, 2000,
3000, 4000 and 5000 in the order listed); decode lengths come from
``default_rng(4004).integers(1024, 32768, size=32, endpoint=True)``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16_NAN_BITS = 0x7FC0


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "fwd" or "decode"
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str  # "bf16" or "f32"
    Nq: int = 0
    Nk: int = 0
    causal: bool = False
    rope_base: float = 0.0
    sigma_qk: float = 1.0
    sigma_v: float = 1.0
    seed_base: int = 0
    # decode only
    max_len: int = 0
    len_lo: int = 0
    len_hi: int = 0
    lens_seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    "f32_n256": Workload("f32_n256", "fwd", B=1, Hq=1, Hkv=1, d=64, dtype="f32", Nq=256, Nk=256,
                   causal=False, seed_base=1000,
                   note="single-head non-causal fp32, N=256, d=64"),
    "mha_d64_n2048": Workload("mha_d64_n2048", "fwd", B=4, Hq=16, Hkv=16, d=64, dtype="bf16", Nq=2048, Nk=2048,
                   causal=True, seed_base=2000,
                   note="MHA causal prefill, B=4, H=16, N=2048, d=64"),
    "gqa_rope_n8192": Workload("gqa_rope_n8192", "fwd", B=2, Hq=32, Hkv=8, d=128, dtype="bf16", Nq=8192, Nk=8192,
                   causal=True, rope_base=10000.0, seed_base=3000,
                   note="GQA causal prefill + RoPE 1e4, B=2, Hq=32, Hkv=8, N=8192, d=128"),
    "decode_b32": Workload("decode_b32", "decode", B=32, Hq=32, Hkv=8, d=128, dtype="bf16",
                   max_len=32768, len_lo=1024, len_hi=32768, lens_seed=4004, seed_base=4000,
                   note="GQA decode, B=32, Hq=32, Hkv=8, d=128, lens ~ U[1024, 32768]"),
    "gqa_rope_n32768": Workload("gqa_rope_n32768", "fwd", B=1, Hq=64, Hkv=8, d=128, dtype="bf16", Nq=32768, Nk=32768,
                   causal=True, rope_base=500000.0, sigma_qk=4.0, seed_base=5000,
                   note="long-context GQA causal prefill + RoPE 5e5, B=1, Hq=64, Hkv=8, "
                        "N=32768, d=128, Q,K ~ N(0,16)"),
}


# ---------------------------------------------------------------- rounding
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------- draws
def normal(shape, seed: int, sigma: float = 1.0, dtype: str = "bf16") -> np.ndarray:
    """Seeded N(0, sigma^2) draw in fp32; bf16 -> uint16 bits, f32 -> float32."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(dtype)


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 values of a stored array (bf16 bits or fp32)."""
    return bf16_bits_to_f64(x) if dtype == "bf16" else np.asarray(x, np.float64)


def fwd_inputs(w: Workload, *, B=None, Hq=None, Hkv=None, Nq=None, Nk=None, d=None,
               seed_base=None):
    """Q, K, V for a prefill workload (optionally with overridden sizes)."""
    B = w.B if B is None else B
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    Nq = w.Nq if Nq is None else Nq
    Nk = w.Nk if Nk is None else Nk
    d = w.d if d is None else d
    s = w.seed_base if seed_base is None else seed_base
    q = normal((B, Hq, Nq, d), s + 1, w.sigma_qk, w.dtype)
    k = normal((B, Hkv, Nk, d), s + 2, w.sigma_qk, w.dtype)
    v = normal((B, Hkv, Nk, d), s + 3, w.sigma_v, w.dtype)
    return q, k, v


def decode_lens(w: Workload, B=None) -> np.ndarray:
    B = w.B if B is None else B
    rng = np.random.default_rng(w.lens_seed)
    return rng.integers(w.len_lo, w.len_hi, size=B, endpoint=True).astype(np.int32)


def decode_inputs(w: Workload, lens: np.ndarray, *, Hq=None, Hkv=None, max_len=None,
                  d=None, seed_base=None, pad_nan: bool = True):
    """q [B,Hq,d] and contiguous caches [B,Hkv,max_len,d] for a decode workload.

    Valid rows 0..len_b-1 of sequence b are drawn per sequence in order from one
    generator per tensor; rows past len_b hold bf16 NaN (so any read past the
    valid length poisons the output) unless ``pad_nan`` is false (then zeros).
    """
    B = len(lens)
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    max_len = w.max_len if max_len is None else max_len
    d = w.d if d is None else d
    s = w.seed_base if seed_base is None else seed_base
    assert w.dtype == "bf16"
    q = normal((B, Hq, d), s + 1, w.sigma_qk, "bf16")
    fill = BF16_NAN_BITS if pad_nan else 0
    kc = np.full((B, Hkv, max_len, d), fill, dtype=np.uint16)
    vc = np.full((B, Hkv, max_len, d), fill, dtype=np.uint16)
    rk = np.random.default_rng(s + 2)
    rv = np.random.default_rng(s + 3)
    for b in range(B):
        n = int(lens[b])
        kb = rk.standard_normal((Hkv, n, d), dtype=np.float32)
        vb = rv.standard_normal((Hkv, n, d), dtype=np.float32)
        if w.sigma_qk != 1.0:
            kb *= np.float32(w.sigma_qk)
        if w.sigma_v != 1.0:
            vb *= np.float32(w.sigma_v)
        kc[b, :, :n] = f32_to_bf16_bits(kb)
        vc[b, :, :n] = f32_to_bf16_bits(vb)
    return q, kc, vc


def paged_inputs(w: Workload, lens: np.ndarray, *, block_size: int = 16, T: int = 1, Hq=None,
                 Hkv=None, d=None, seed_base=None, spare_blocks: int = 8, max_blocks=None):
    """q [B,Hq,T,d], K/V pools [num_blocks,Hkv,block_size,d] (bf16 bits) and an
    int32 block table [B, max_blocks] for a paged decode workload.

    Sequence b owns ceil(len_b / block_size) physical blocks taken in order from
    one seeded permutation of the pool (so logically adjacent blocks sit at
    unrelated physical places); ``spare_blocks`` more blocks stay unowned.  Its
    rows are drawn per sequence in order from one generator per tensor, with
    the same distribution as ``decode_inputs``.  Every pool row that no sequence
    owns (spare blocks and the tail of each last block) holds bf16 NaN, and
    table entries past a sequence's blocks are -1.
    """
    B = len(lens)
    Hq = w.Hq if Hq is None else Hq
    Hkv = w.Hkv if Hkv is None else Hkv
    d = w.d if d is None else d
    s = w.seed_base if seed_base is None else seed_base
    bs = block_size
    nb = [(int(n) + bs - 1) // bs for n in lens]
    mb = max(nb + [1]) if max_blocks is None else max_blocks
    num_blocks = sum(nb) + spare_blocks
    perm = np.random.default_rng(s + 5).permutation(num_blocks).astype(np.int32)
    table = np.full((B, mb), -1, dtype=np.int32)
    kp = np.full((num_blocks, Hkv, bs, d), BF16_NAN_BITS, dtype=np.uint16)
    vp = np.full((num_blocks, Hkv, bs, d), BF16_NAN_BITS, dtype=np.uint16)
    q = normal((B, Hq, T, d), s + 1, w.sigma_qk, "bf16")
    rk = np.random.default_rng(s + 2)
    rv = np.random.default_rng(s + 3)
    off = 0
    for b in range(B):
        n = int(lens[b])
        phys = perm[off:off + nb[b]]
        off += nb[b]
        table[b, :nb[b]] = phys
        for pool, r, sig in ((kp, rk, w.sigma_qk), (vp, rv, w.sigma_v)):
            x = r.standard_normal((Hkv, n, d), dtype=np.float32)
            if sig != 1.0:
                x *= np.float32(sig)
            full = np.full((Hkv, nb[b] * bs, d), BF16_NAN_BITS, dtype=np.uint16)
            full[:, :n] = f32_to_bf16_bits(x)
            pool[phys] = full.reshape(Hkv, nb[b], bs, d).transpose(1, 0, 2, 3)
    return q, kp, vp, table
