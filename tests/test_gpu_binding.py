"""The Python binding rejects caller-supplied tensors the kernels could not
write safely (wrong shape, dtype, layout or device) before anything is
launched, and a workspace that is too small is refused by the library itself.
Valid calls with and without the optional lse agree with each other."""

import math

import numpy as np
import pytest

import workloads as W
from gpu_util import dev, host

pytestmark = pytest.mark.gpu

esd = pytest.importorskip("exact_scaled_dot_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    esd.lib()
    yield
    torch.cuda.synchronize()


def _fwd_inputs(B=1, Hq=4, Hkv=2, N=100, d=64):
    q = dev(W.normal((B, Hq, N, d), 12001, 1.0, "bf16"))
    k = dev(W.normal((B, Hkv, N, d), 12002, 1.0, "bf16"))
    v = dev(W.normal((B, Hkv, N, d), 12003, 1.0, "bf16"))
    return q, k, v


def test_fwd_rejects_bad_outputs():
    import torch
    q, k, v = _fwd_inputs()
    f32 = dict(dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):  # too small
        esd.fwd(q, k, v, True, out=torch.empty((1, 4, 99, 64), **f32))
    with pytest.raises(TypeError):  # wrong dtype
        esd.fwd(q, k, v, True, out=torch.empty((1, 4, 100, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):  # not contiguous
        esd.fwd(q, k, v, True, out=torch.empty((1, 4, 64, 100), **f32).transpose(2, 3))
    with pytest.raises(ValueError):  # on the host
        esd.fwd(q, k, v, True, out=torch.empty((1, 4, 100, 64), dtype=torch.float32))
    with pytest.raises(ValueError):
        esd.fwd(q, k, v, True, lse=torch.empty((1, 4, 64), **f32))
    with pytest.raises(TypeError):  # workspace must be bytes
        esd.fwd(q, k, v, True, rope_base=1e4, workspace=torch.empty(100 * 64, **f32))
    with pytest.raises(ValueError):  # inputs on the host
        esd.fwd(q.cpu(), k, v, True)


def test_fwd_small_workspace_is_refused():
    import torch
    q, k, v = _fwd_inputs()
    need = esd.fwd_workspace_bytes(1, 2, 100, 64, 1e4, esd.ATTN_BF16)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(esd.AttnError) as e:
        esd.fwd(q, k, v, True, rope_base=1e4, workspace=ws)
    assert e.value.code == 4  # ATTN_ERR_WORKSPACE


def test_fwd_without_lse_matches():
    import torch
    q, k, v = _fwd_inputs()
    o1, l1 = esd.fwd(q, k, v, True, rope_base=1e4)
    o2, l2 = esd.fwd(q, k, v, True, rope_base=1e4, want_lse=False)
    torch.cuda.synchronize()
    assert l2 is None
    assert np.array_equal(host(o1), host(o2))


def test_bwd_rejects_bad_gradients():
    import torch
    q, k, v = _fwd_inputs()
    o, lse = esd.fwd(q, k, v, True)
    do = torch.ones_like(o)
    f32 = dict(dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):  # dk with the query head count
        esd.bwd(q, k, v, o, lse, do, True, dk=torch.empty((1, 4, 100, 64), **f32))
    with pytest.raises(TypeError):
        esd.bwd(q, k, v, o, lse, do, True, dq=torch.empty((1, 4, 100, 64), dtype=torch.float64,
                                                          device="cuda"))
    torch.cuda.synchronize()


def test_decode_rejects_bad_outputs():
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.array([5, 300, 1500], dtype=np.int32)
    q, kc, vc = W.decode_inputs(w, lens, Hq=8, Hkv=2, d=64, max_len=1600, seed_base=12100)
    f32 = dict(dtype=torch.float32, device="cuda")
    args = (dev(q), dev(kc), dev(vc), dev(lens))
    with pytest.raises(ValueError):
        esd.decode(*args, out=torch.empty((3, 8, 128), **f32))
    with pytest.raises(ValueError):
        esd.decode(*args, lse=torch.empty((8, 3), **f32))
    with pytest.raises(TypeError):
        esd.decode(*args, workspace=torch.empty(10, dtype=torch.int32, device="cuda"))
    with pytest.raises(esd.AttnError) as e:
        esd.decode(*args, workspace=torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.code == 4
    o1, l1 = esd.decode(*args)
    o2, _ = esd.decode(*args, want_lse=False)
    torch.cuda.synchronize()
    assert np.array_equal(host(o1), host(o2))


def test_decode_multi_rejects_wrong_token_count():
    import torch
    w = W.WORKLOADS["decode_b32"]
    lens = np.array([40, 300], dtype=np.int32)
    _, kc, vc = W.decode_inputs(w, lens, Hq=8, Hkv=2, d=64, max_len=512, seed_base=12200)
    q = W.normal((2, 8, 2, 64), 12207, 1.0, "bf16")
    with pytest.raises(ValueError):
        esd.decode_multi(dev(q), dev(kc), dev(vc), dev(lens),
                         out=torch.empty((2, 8, 1, 64), dtype=torch.float32, device="cuda"))
    o, l = esd.decode_multi(dev(q), dev(kc), dev(vc), dev(lens), scale=1 / math.sqrt(64))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(o))) and np.all(np.isfinite(host(l)))


def test_rope_apply_rejects_bad_output():
    import torch
    x = dev(W.normal((1, 2, 10, 64), 12300, 1.0, "bf16"))
    with pytest.raises(TypeError):
        esd.rope_apply(x, 1e4, out=torch.empty((1, 2, 10, 64), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        esd.rope_apply(x, 1e4, out=torch.empty((1, 2, 9, 64), dtype=torch.bfloat16, device="cuda"))
