"""The entry points queue their work and return: after a call with a long
kernel (the N = 32768 forward takes about 16 ms, the N = 8192 backward about
3.5 ms), an event recorded right after the call has not completed yet.  The
inputs are random device tensors; the results are checked elsewhere."""

import math

import pytest

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


def _rand(shape):
    import torch
    return torch.randn(shape, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def test_forward_returns_before_the_kernel_ends():
    import torch
    q, k, v = _rand((1, 64, 32768, 128)), _rand((1, 8, 32768, 128)), _rand((1, 8, 32768, 128))
    esd.fwd(q, k, v, True, 1 / math.sqrt(128))  # first call: library and output allocation
    torch.cuda.synchronize()
    o, lse = esd.fwd(q, k, v, True, 1 / math.sqrt(128))
    done = torch.cuda.Event()
    done.record()
    assert not done.query(), "attn_fwd waited for its kernel"
    torch.cuda.synchronize()
    assert done.query()


def test_backward_returns_before_the_kernels_end():
    import torch
    B, Hq, Hkv, N, d = 2, 32, 8, 8192, 128
    q, k, v = _rand((B, Hq, N, d)), _rand((B, Hkv, N, d)), _rand((B, Hkv, N, d))
    o, lse = esd.fwd(q, k, v, True, 1 / math.sqrt(d), 1e4)
    do = torch.randn((B, Hq, N, d), device="cuda", dtype=torch.float32)
    esd.bwd(q, k, v, o, lse, do, causal=True, scale=1 / math.sqrt(d), rope_base=1e4)
    torch.cuda.synchronize()
    esd.bwd(q, k, v, o, lse, do, causal=True, scale=1 / math.sqrt(d), rope_base=1e4)
    done = torch.cuda.Event()
    done.record()
    assert not done.query(), "attn_bwd waited for its kernels"
    torch.cuda.synchronize()
    assert done.query()
