"""Host dispatch checks that need the stand-in runtime of stubs.cpp: run only by
run.py against the sanitizer build (not collected in the normal test run).

Device pointers here are fake addresses the stubs never dereference; the
RoPE table, whose "device" memory is host memory under the stubs, is read back
and compared with Python's math module (the same C library).
"""

import ctypes
import math

import pytest

import exact_scaled_dot_amd as esd

BF16, F32 = esd.ATTN_BF16, esd.ATTN_F32
PREFILL_BF16, PREFILL_F32, ROPE_BF16, ROPE_F32, DECODE, BWD, SCRATCH = range(7)


@pytest.fixture()
def L():
    lib = esd.lib()
    vp = ctypes.c_void_p
    for name in ("stub_fwd_k", "stub_fwd_rope_tab", "stub_dec_ws_o", "stub_dec_ws_lse",
                 "stub_dec_rope_tab", "stub_bwd_q", "stub_bwd_k", "stub_scratch", "stub_rope_out"):
        getattr(lib, name).restype = vp
    lib.stub_rope_out.argtypes = [ctypes.c_int]
    lib.stub_calls.argtypes = [ctypes.c_int]
    lib.stub_set_capturing.argtypes = [ctypes.c_int]
    lib.stub_reset()
    lib.stub_set_capturing(0)
    yield lib
    lib.stub_set_capturing(0)


def A(x):
    return ctypes.c_void_p(x)


Q, K, V, O, LSE, WS = (A(0x100000 * (i + 1)) for i in range(6))


STREAM = A(0x1234)  # a fake non-null stream (the null stream is never captured)


def _fwd(L, rope, Nk=300, ws=WS, wsb=1 << 30, d=128):
    return L.attn_fwd(Q, K, V, O, LSE, 1, 8, 2, 100, Nk, d, 1, 0.1, rope, BF16, ws, wsb, STREAM)


def test_fwd_with_rope_rotates_k_into_the_workspace(L):
    assert _fwd(L, 10000.0) == 0
    assert L.stub_calls(ROPE_BF16) == 1 and L.stub_calls(PREFILL_BF16) == 1
    assert L.stub_fwd_k() == WS.value and L.stub_rope_out(0) == WS.value
    assert L.stub_fwd_rope_tab() is not None and L.stub_fwd_o_bf16() == 0


def test_fwd_without_rope_uses_k_as_given(L):
    assert _fwd(L, 0.0, ws=None, wsb=0) == 0
    assert L.stub_calls(ROPE_BF16) == 0 and L.stub_fwd_k() == K.value
    assert L.stub_fwd_rope_tab() is None


def test_window_covering_every_key_is_plain_causal(L):
    args = (Q, K, V, O, LSE, 1, 8, 2, 100, 300, 128)
    assert L.attn_fwd_window(*args, 50, 0.1, 0.0, BF16, None, 0, None) == 0
    assert L.stub_fwd_window() == 50
    assert L.attn_fwd_window(*args, 300, 0.1, 0.0, BF16, None, 0, None) == 0
    assert L.stub_fwd_window() == 0


def test_prefill_cached_rotates_only_queries(L):
    assert L.attn_prefill_cached(Q, K, V, O, LSE, 1, 8, 2, 100, 300, 128, 0.1, 10000.0, BF16,
                                 BF16, None) == 0
    assert L.stub_calls(ROPE_BF16) == 0 and L.stub_calls(PREFILL_BF16) == 1
    assert L.stub_fwd_k() == K.value and L.stub_fwd_rope_tab() is not None
    assert L.stub_fwd_o_bf16() == 1
    assert L.attn_prefill_cached(Q, K, V, O, LSE, 1, 8, 2, 100, 300, 128, 0.1, 0.0, F32, F32,
                                 None) == 0
    assert L.stub_calls(PREFILL_F32) == 1 and L.stub_fwd_o_bf16() == 0


def _table_value(ptr, pos, j, half):
    cs = (ctypes.c_double * 2).from_address(ptr + 16 * (pos * half + j))
    return cs[0], cs[1]


@pytest.mark.parametrize("base,d", [(10000.0, 128), (500000.0, 64), (10.0, 128)])
def test_rope_table_values_are_the_c_library_values(L, base, d):
    assert _fwd(L, base, Nk=3000, d=d) == 0
    tab = L.stub_fwd_rope_tab()
    half = d // 2
    for pos in (0, 1, 2, 1023, 1024, 2999, 4095):   # the table covers 4096 positions
        for j in (0, 1, half // 2, half - 1):
            ang = float(pos) * math.pow(base, -2.0 * j / d)
            c, s = _table_value(tab, pos, j, half)
            assert c == math.cos(ang) and s == math.sin(ang), (pos, j)


def test_rope_table_grows_and_keeps_the_old_one(L):
    assert _fwd(L, 777.0, Nk=1000) == 0
    small = L.stub_fwd_rope_tab()
    assert _fwd(L, 777.0, Nk=500) == 0 and L.stub_fwd_rope_tab() == small
    assert _fwd(L, 777.0, Nk=1500) == 0
    big = L.stub_fwd_rope_tab()
    assert big != small
    # the old table is still readable (kernels queued earlier may use it)
    assert _table_value(small, 10, 0, 64) == _table_value(big, 10, 0, 64)


def test_rope_table_is_not_built_during_capture(L):
    L.stub_set_capturing(1)
    assert _fwd(L, 4321.0, Nk=100) == 3         # a new table would need blocking copies
    L.stub_set_capturing(0)
    assert _fwd(L, 4321.0, Nk=100) == 0         # built outside capture
    L.stub_set_capturing(1)
    assert _fwd(L, 4321.0, Nk=100) == 0         # and then usable while capturing
    assert _fwd(L, 4321.0, Nk=5000) == 3        # but not grown


def test_decode_workspace_split(L):
    B, Hq, Hkv, T, max_len, d = 3, 8, 2, 2, 5000, 128
    need = esd.decode_multi_workspace_bytes(B, Hq, Hkv, T, max_len, d)
    ws = A(0x4000000)
    assert L.attn_decode_multi(Q, K, V, A(0x7000000), O, LSE, B, Hq, Hkv, T, max_len, d, 0.1,
                               10000.0, BF16, BF16, ws, need, None) == 0
    nch = (max_len + 2047) // 2048
    rows = B * Hq * T * nch
    o_bytes = (rows * d * 4 + 255) // 256 * 256
    assert L.stub_dec_nchunks() == nch and L.stub_dec_ws_o() == ws.value
    assert L.stub_dec_ws_lse() == ws.value + o_bytes
    assert o_bytes + rows * 4 == need and L.stub_dec_o_bf16() == 1
    assert L.stub_dec_rope_tab() is not None


def test_decode_noalloc_uses_the_static_array(L):
    assert L.attn_decode_noalloc(Q, K, V, A(0x7000000), O, LSE, 4, 8, 2, 5000, 128, 0.1, BF16,
                                 None) == 0
    assert L.stub_calls(SCRATCH) == 1 and L.stub_dec_ws_o() == L.stub_scratch()


def test_bwd_with_rope_rotates_q_and_k(L):
    need = esd.bwd_workspace_bytes(1, 8, 2, 100, 300, 128, 1e4, BF16)
    ws = A(0x40000000)
    assert L.attn_bwd(Q, K, V, O, LSE, A(0x800000), A(0x900000), A(0xa00000), A(0xb00000), 1, 8, 2,
                      100, 300, 128, 1, 0.1, 1e4, BF16, ws, need, None) == 0
    assert L.stub_calls(ROPE_BF16) == 2 and L.stub_calls(BWD) == 1
    assert L.stub_bwd_q() == L.stub_rope_out(0) and L.stub_bwd_k() == L.stub_rope_out(1)
