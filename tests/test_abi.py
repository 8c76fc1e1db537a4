"""The C-ABI library loads, exports what include/attn.h declares, and rejects
invalid arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

import exact_scaled_dot_amd as esd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(esd.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = esd.lib()
    for name in _declared():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_status_strings():
    for code, name in esd.STATUS.items():
        assert esd.status_str(code) == name
    assert esd.status_str(99) == "ATTN_ERR_UNKNOWN"


def test_workspace_sizes():
    assert esd.fwd_workspace_bytes(2, 8, 8192, 128, 0.0, esd.ATTN_BF16) == 0
    assert esd.fwd_workspace_bytes(2, 8, 8192, 128, 10000.0, esd.ATTN_BF16) == 2 * 8 * 8192 * 128 * 2
    assert esd.fwd_workspace_bytes(1, 1, 256, 64, 100.0, esd.ATTN_F32) == 256 * 64 * 4
    n = esd.decode_workspace_bytes(32, 32, 8, 32768, 128)
    rows = 32 * 32 * (32768 // 2048)  # one partial state per 2048-key chunk
    assert n >= rows * 129 * 4 and n < rows * 129 * 4 + 256
    assert esd.decode_workspace_bytes(0, 32, 8, 32768, 128) == 0


P = ctypes.c_void_p(256)  # a non-null, aligned, never dereferenced address


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=64, causal=1,
             scale=0.125, rope=0.0, dtype=esd.ATTN_BF16, ws=None, wsb=0)
    a.update(kw)
    return esd.lib().attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"], a["rope"],
                              a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(B=-1), 1), (dict(Hkv=0), 1),
    (dict(Hq=6, Hkv=4), 1), (dict(causal=2), 1), (dict(Nq=9, Nk=8), 1),
    (dict(Nk=0), 1), (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1), (dict(scale=0.0), 1),
    (dict(scale=-0.5), 1),
    (dict(rope=-1.0), 1), (dict(rope=float("inf")), 1), (dict(dtype=7), 1),
    (dict(d=96), 2), (dict(d=32), 2), (dict(q=ctypes.c_void_p(258)), 1),
    (dict(rope=10000.0), 4), (dict(rope=10000.0, ws=P, wsb=100), 4),
    (dict(causal=0, Nq=9, Nk=8, rope=100.0, ws=P, wsb=1 << 20), 1),  # negative RoPE positions
])
def test_fwd_rejects_on_host(kw, code):
    assert _fwd(**kw) == code


def _fwd_window(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=64, window=4,
             scale=0.125, rope=0.0, dtype=esd.ATTN_BF16, ws=None, wsb=0)
    a.update(kw)
    return esd.lib().attn_fwd_window(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                     a["Hkv"], a["Nq"], a["Nk"], a["d"], a["window"], a["scale"],
                                     a["rope"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=0), 1), (dict(window=-3), 1), (dict(Nq=9, Nk=8), 1), (dict(v=None), 1),
    (dict(d=80), 2), (dict(scale=0.0), 1), (dict(rope=100.0), 4),
])
def test_fwd_window_rejects_on_host(kw, code):
    assert _fwd_window(**kw) == code


def test_fwd_window_empty_is_a_noop():
    assert _fwd_window(q=None, k=None, v=None, o=None, Nq=0) == 0


@pytest.mark.parametrize("kw", [dict(B=0), dict(Hq=0, Hkv=1), dict(Nq=0)])
def test_fwd_empty_is_a_noop(kw):
    assert _fwd(q=None, k=None, v=None, o=None, **kw) == 0


def _pfc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=None, B=1, Hq=4, Hkv=2, Nq=8, Nk=8, d=64, scale=0.125,
             rope=0.0, dtype=esd.ATTN_BF16, odt=esd.ATTN_F32)
    a.update(kw)
    return esd.lib().attn_prefill_cached(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                         a["Hkv"], a["Nq"], a["Nk"], a["d"], a["scale"], a["rope"],
                                         a["dtype"], a["odt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(Hq=6, Hkv=4), 1), (dict(Nq=9, Nk=8), 1),
    (dict(Nk=0), 1), (dict(scale=0.0), 1), (dict(rope=-1.0), 1), (dict(dtype=7), 1),
    (dict(odt=2), 1), (dict(d=96), 2), (dict(o=ctypes.c_void_p(264)), 1),
])
def test_prefill_cached_rejects_on_host(kw, code):
    assert _pfc(**kw) == code


def test_prefill_cached_empty_is_a_noop():
    assert _pfc(q=None, k=None, v=None, o=None, Nq=0) == 0


def _dec(**kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, max_len=64, d=128,
             scale=0.1, dtype=esd.ATTN_BF16, ws=P, wsb=1 << 20)
    a.update(kw)
    return esd.lib().attn_decode(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"],
                                 a["Hq"], a["Hkv"], a["max_len"], a["d"], a["scale"], a["dtype"],
                                 a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lens=None), 1), (dict(k=None), 1), (dict(Hq=6, Hkv=4), 1), (dict(max_len=0), 1),
    (dict(scale=float("nan")), 1), (dict(scale=-1.0), 1), (dict(dtype=esd.ATTN_F32), 2), (dict(d=80), 2),
    (dict(ws=None), 4), (dict(wsb=10), 4), (dict(ws=ctypes.c_void_p(272)), 1),
    (dict(max_len=1 << 23), 2),
])
def test_decode_rejects_on_host(kw, code):
    assert _dec(**kw) == code


def _dec_noalloc(**kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, max_len=64, d=128,
             scale=0.1, dtype=esd.ATTN_BF16)
    a.update(kw)
    return esd.lib().attn_decode_noalloc(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"],
                                         a["B"], a["Hq"], a["Hkv"], a["max_len"], a["d"],
                                         a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lens=None), 1), (dict(k=None), 1), (dict(Hq=6, Hkv=4), 1), (dict(max_len=0), 1),
    (dict(scale=float("nan")), 1), (dict(dtype=esd.ATTN_F32), 2), (dict(d=80), 2),
    (dict(q=ctypes.c_void_p(258)), 1), (dict(max_len=1 << 23), 2),
    # partial states past the static array: 64 * 32 rows x 17 chunks of 2048 keys
    (dict(B=64, Hq=32, Hkv=8, max_len=34000), 4),
])
def test_decode_noalloc_rejects_on_host(kw, code):
    assert _dec_noalloc(**kw) == code


def test_decode_noalloc_limit_matches_workspace_sizes():
    assert esd.decode_workspace_bytes(32, 32, 8, 32768, 128) <= esd.DECODE_NOALLOC_MAX_BYTES
    assert esd.decode_workspace_bytes(64, 32, 8, 34000, 128) > esd.DECODE_NOALLOC_MAX_BYTES
    hdr = open(os.path.join(ROOT, "include", "attn.h")).read()
    assert "#define ATTN_DECODE_NOALLOC_MAX_BYTES ((size_t)16 << 20)" in hdr
    assert esd.DECODE_NOALLOC_MAX_BYTES == 16 << 20
    assert _dec_noalloc(B=0, q=None, k=None, v=None, lens=None, o=None) == 0


def test_decode_empty_is_a_noop():
    assert _dec(B=0, q=None, k=None, v=None, lens=None, o=None, ws=None, wsb=0) == 0


def _decm(**kw):
    a = dict(q=P, k=P, v=P, lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, T=4, max_len=64, d=128,
             scale=0.1, rope=0.0, dtype=esd.ATTN_BF16, odt=esd.ATTN_F32, ws=P, wsb=1 << 20)
    a.update(kw)
    return esd.lib().attn_decode_multi(a["q"], a["k"], a["v"], a["lens"], a["o"], a["lse"], a["B"],
                                       a["Hq"], a["Hkv"], a["T"], a["max_len"], a["d"], a["scale"],
                                       a["rope"], a["dtype"], a["odt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), 1), (dict(T=-2), 1), (dict(lens=None), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(scale=0.0), 1), (dict(rope=-5.0), 1), (dict(rope=float("nan")), 1),
    (dict(dtype=esd.ATTN_F32), 2), (dict(d=96), 2), (dict(ws=None), 4), (dict(wsb=100), 4),
    (dict(ws=ctypes.c_void_p(272)), 1), (dict(B=1 << 12, Hq=1 << 12, Hkv=1, T=1 << 8), 2),
    (dict(odt=5), 1), (dict(odt=-1), 1),
])
def test_decode_multi_rejects_on_host(kw, code):
    assert _decm(**kw) == code


def test_decode_multi_workspace():
    one = esd.decode_workspace_bytes(3, 8, 2, 5000, 128)
    assert esd.decode_multi_workspace_bytes(3, 8, 2, 1, 5000, 128) == one
    rows = 3 * 8 * 6 * 3  # B * Hq * T * chunks of 2048 keys
    n = esd.decode_multi_workspace_bytes(3, 8, 2, 6, 5000, 128)
    assert rows * 129 * 4 <= n < rows * 129 * 4 + 256
    assert esd.decode_multi_workspace_bytes(3, 8, 2, 0, 5000, 128) == 0


def _decp(**kw):
    a = dict(q=P, k=P, v=P, table=P, lens=P, o=P, lse=None, B=2, Hq=8, Hkv=2, T=1, nblk=64,
             bs=16, mb=8, d=128, scale=0.1, rope=0.0, dtype=esd.ATTN_BF16, odt=esd.ATTN_F32, ws=P,
             wsb=1 << 20)
    a.update(kw)
    return esd.lib().attn_decode_paged(a["q"], a["k"], a["v"], a["table"], a["lens"], a["o"],
                                       a["lse"], a["B"], a["Hq"], a["Hkv"], a["T"], a["nblk"],
                                       a["bs"], a["mb"], a["d"], a["scale"], a["rope"], a["dtype"],
                                       a["odt"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(table=None), 1), (dict(nblk=0), 1), (dict(mb=0), 1), (dict(bs=8), 2), (dict(bs=24), 2),
    (dict(bs=8192), 2), (dict(mb=1 << 20, bs=4096), 2), (dict(T=0), 1), (dict(lens=None), 1),
    (dict(dtype=esd.ATTN_F32), 2), (dict(ws=None), 4), (dict(d=80), 2), (dict(odt=3), 1),
])
def test_decode_paged_rejects_on_host(kw, code):
    assert _decp(**kw) == code


def test_decode_paged_workspace_and_noop():
    assert (esd.decode_paged_workspace_bytes(3, 8, 2, 2, 20, 16, 128)
            == esd.decode_multi_workspace_bytes(3, 8, 2, 2, 320, 128))
    # 3200 keys: a paged cache is split into chunks of 1024 keys (4 partial
    # states per row), a contiguous one into chunks of 2048 (2 per row)
    rows_paged, rows_contig = 3 * 8 * 2 * 4, 3 * 8 * 2 * 2
    n = esd.decode_paged_workspace_bytes(3, 8, 2, 2, 200, 16, 128)
    assert rows_paged * 129 * 4 <= n < rows_paged * 129 * 4 + 256
    n = esd.decode_multi_workspace_bytes(3, 8, 2, 2, 3200, 128)
    assert rows_contig * 129 * 4 <= n < rows_contig * 129 * 4 + 256
    assert esd.decode_paged_workspace_bytes(3, 8, 2, 2, 1 << 20, 1 << 12, 128) == 0
    assert _decp(B=0, q=None, k=None, v=None, table=None, lens=None, o=None, ws=None, wsb=0) == 0


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, B=1, Hq=4, Hkv=2, Nq=8, Nk=8,
             d=128, causal=1, scale=0.1, rope=0.0, dtype=esd.ATTN_BF16, ws=P, wsb=1 << 20)
    a.update(kw)
    return esd.lib().attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                              a["dv"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nk"], a["d"],
                              a["causal"], a["scale"], a["rope"], a["dtype"], a["ws"], a["wsb"],
                              None)


@pytest.mark.parametrize("kw,code", [
    (dict(dq=None), 1), (dict(lse=None), 1), (dict(do=None), 1), (dict(Nq=9, Nk=8), 1),
    (dict(causal=0, Nq=9, Nk=8, rope=100.0), 1), (dict(causal=3), 1), (dict(scale=-1.0), 1),
    (dict(dtype=esd.ATTN_F32), 2), (dict(d=96), 2), (dict(ws=None), 4), (dict(wsb=64), 4),
    (dict(ws=ctypes.c_void_p(272)), 1), (dict(dk=ctypes.c_void_p(260)), 1),
])
def test_bwd_rejects_on_host(kw, code):
    assert _bwd(**kw) == code


def test_bwd_workspace():
    rows = 2 * 8 * 100
    base = esd.bwd_workspace_bytes(2, 8, 2, 100, 300, 128, 0.0, esd.ATTN_BF16)
    assert rows * 128 * 2 + 2 * rows * 4 <= base < rows * 128 * 2 + 2 * rows * 4 + 3 * 256
    rope = esd.bwd_workspace_bytes(2, 8, 2, 100, 300, 128, 1e4, esd.ATTN_BF16)
    assert rope - base >= rows * 128 * 2 + 2 * 2 * 300 * 128 * 2
    assert esd.bwd_workspace_bytes(2, 8, 2, 100, 300, 128, 0.0, esd.ATTN_F32) == 0
    assert _bwd(B=0, q=None, k=None, v=None, o=None, lse=None, do=None, dq=None, dk=None,
                dv=None, ws=None, wsb=0) == 0


def test_decode_multi_empty_is_a_noop():
    assert _decm(B=0, q=None, k=None, v=None, lens=None, o=None, ws=None, wsb=0) == 0


def test_rope_apply_rejects_on_host():
    L = esd.lib()
    assert L.attn_rope_apply(P, P, 1, 1, 4, 7, 0, 100.0, esd.ATTN_BF16, None) == 1
    assert L.attn_rope_apply(P, P, 1, 1, 4, 12, 0, 100.0, esd.ATTN_BF16, None) == 2
    assert L.attn_rope_apply(P, P, 1, 1, 4, 16, 0, 0.0, esd.ATTN_BF16, None) == 1
    assert L.attn_rope_apply(None, P, 1, 1, 4, 16, 0, 100.0, esd.ATTN_BF16, None) == 1
    assert L.attn_rope_apply(None, None, 0, 1, 4, 16, 0, 100.0, esd.ATTN_BF16, None) == 0
    # positions past 2^22 (the RoPE table's limit) are refused before any HIP call
    assert L.attn_rope_apply(P, P, 1, 1, 4, 16, (1 << 22) - 3, 100.0, esd.ATTN_BF16, None) == 2
    assert L.attn_rope_apply(P, P, 1, 1, 4, 16, 1 << 30, 100.0, esd.ATTN_BF16, None) == 2


def test_rope_positions_past_the_table_limit_rejected():
    # d = 64 allows 5M keys per head, but RoPE positions stop at 2^22
    assert _fwd(Nq=8, Nk=5 << 20, rope=100.0, ws=P, wsb=1 << 40) == 2
    assert _decm(max_len=5 << 20, d=64, rope=100.0) == 2
    assert _pfc(Nq=8, Nk=5 << 20, rope=100.0) == 2
