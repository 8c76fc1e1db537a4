"""Helpers for the GPU tests: move seeded numpy inputs to the device and compare."""

import sys

import numpy as np


def dev(x):
    """numpy uint16 (bf16 bits) / float32 / int32 array -> contiguous cuda tensor."""
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def max_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


TOL = {"bf16": (1e-2, 1e-3), "f32": (1e-4, 1e-4)}


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    to, tl = TOL[dtype]
    eo = max_err(o_gpu, o_ref)
    el = max_err(lse_gpu, lse_ref)
    say(f"{what}: max|dO|={eo:.3e} (tol {to}), max|dlse|={el:.3e} (tol {tl})")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), what
    assert eo <= to, (what, eo)
    assert el <= tl, (what, el)


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (2^(e - 7) for |x| in [2^e, 2^(e+1)))."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_bf16_o(o_gpu, lse_gpu, o_ref, lse_ref, what=""):
    """A bf16 O against the oracle's O rounded the same way (fp64 -> fp32 ->
    bf16, nearest even): within the bf16 tolerance on the unrounded value plus
    one bf16 spacing, since the two sides round values up to 1e-2 apart; lse
    is fp32 and keeps its own tolerance."""
    import oracle.dense as oa
    to, tl = TOL["bf16"]
    o_ref_r = oa.round_to_dtype(o_ref, "bf16")
    err = np.abs(np.asarray(o_gpu, np.float64) - o_ref_r)
    lim = to + bf16_ulp(o_ref)
    eo = float(np.max(err)) if err.size else 0.0
    el = max_err(lse_gpu, lse_ref)
    say(f"{what}: bf16 O max|dO|={eo:.3e} (tol {to} + 1 bf16 spacing), max|dlse|={el:.3e} (tol {tl})")
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), what
    assert np.all(err <= lim), (what, eo)
    assert el <= tl, (what, el)
