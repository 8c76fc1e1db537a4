"""Randomised arguments for every entry point, run only by run.py against the
sanitizer build of the host code (not collected in the normal test run).

Sizes are drawn from edge values (negative, 0, 1, tile edges, 2^31 - 1) and
small ranges, together with unknown enum values, non-finite scales and bases,
NULL or fake device pointers and workspaces of 0 bytes to 1 TiB.  Every call
must return one of the status codes the header defines, and every
workspace-size query the exact size, or SIZE_MAX where that does not fit in
size_t.  AddressSanitizer and
UndefinedBehaviorSanitizer (which stops at the first signed overflow, invalid
shift or out-of-bounds access) watch every call.  The stand-in runtime never
touches the fake pointers.  The one host allocation a call can make is the
RoPE table, which the stubs really build: with a valid RoPE base the sizes
that set its length stay below 4096 positions.
"""

import ctypes
import math

from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import exact_scaled_dot_amd as esd

CODES = {0, 1, 2, 3, 4}
SIZE_MAX = (1 << 64) - 1


CHUNK, CHUNK_PAGED = 2048, 1024  # keys per split-decode workgroup (contiguous, paged)


def _sat(x):
    # the size as it must come back: exact, or SIZE_MAX where it does not fit
    return x if x <= SIZE_MAX else SIZE_MAX


def _a256(x):
    return (x + 255) // 256 * 256


def fwd_ws(B, Hkv, Nk, d, rb, dt):
    if not rb > 0 or min(B, Hkv, Nk, d) <= 0 or dt not in (0, 1):
        return 0
    return _sat(B * Hkv * Nk * d * (4 if dt == 1 else 2))


def dec_ws(B, Hq, Hkv, T, max_len, d, chunk):
    if min(B, Hq, Hkv, T, max_len, d) <= 0:
        return 0
    rows = B * Hq * T * (-(-max_len // chunk))
    return _sat(_a256(rows * d * 4) + rows * 4)


def bwd_ws(B, Hq, Hkv, Nq, Nk, d, rb, dt):
    if min(B, Hq, Hkv, Nq, Nk, d) <= 0 or dt != 0:
        return 0
    rows = B * Hq * Nq
    n = _a256(rows * d * 2) + 2 * _a256(rows * 4)
    if rb > 0:
        n += _a256(rows * d * 2) + _a256(B * Hkv * Nk * d * 2)
    return _sat(n)
EDGE = [-(1 << 31), -1, 0, 1, 2, 7, 31, 32, 33, 63, 64, 65, 255, 256, 257, 4095, 4096,
        1 << 20, (1 << 22) - 1, 1 << 22, (1 << 30), (1 << 31) - 1]
size = st.one_of(st.sampled_from(EDGE), st.integers(-3, 600))
small = st.one_of(st.sampled_from([-1, 0, 1, 2, 3, 4, 8, 16, 64, 1 << 16, (1 << 31) - 1]),
                  st.integers(1, 40))
dims = st.sampled_from([-1, 0, 2, 8, 16, 64, 100, 128, 256, 512, 520])
dtype = st.sampled_from([-1, 0, 1, 2])
flag = st.sampled_from([-1, 0, 1, 2])
scale = st.sampled_from([0.1, 1.0, 0.0, -1.0, 1e-30, 1e30, math.inf, -math.inf, math.nan])
base = st.sampled_from([0.0, 1e4, 5e5, 0.5, 1.0, -1.0, math.inf, math.nan])
wsb = st.sampled_from([0, 1, 255, 1 << 20, 1 << 40])
ptr = st.sampled_from([0, 1, 2, 3])  # 0 = NULL, else a fake 16-byte-aligned address
MAXPOS = 4096

SETTINGS = settings(max_examples=300, deadline=None, derandomize=True,
                    suppress_health_check=list(HealthCheck))


def P(k, slot=0):
    return None if k == 0 else ctypes.c_void_p(0x1000000 * (k + 4 * slot))


def S(k):
    return None if k == 0 else ctypes.c_void_p(0x4321)


def rope_ok(b):
    return math.isfinite(b) and b > 1.0


def cap(n, b):
    # keep the RoPE table short when the base is valid (the stubs build it)
    return min(n, MAXPOS) if rope_ok(b) else n


def L():
    lib = esd.lib()
    lib.stub_set_capturing(0)
    return lib


@SETTINGS
@given(st.tuples(small, small, small, size, size, dims, flag, scale, base, dtype, ptr, wsb, ptr, ptr))
def test_fwd(a):
    B, Hq, Hkv, Nq, Nk, d, causal, sc, rb, dt, p, nb, w, strm = a
    Nk = cap(Nk, rb)
    lib = L()
    r = lib.attn_fwd(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), B, Hq, Hkv, Nq, Nk, d, causal,
                     sc, rb, dt, P(w, 5), nb, S(strm))
    assert r in CODES
    r = lib.attn_fwd_window(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), B, Hq, Hkv, Nq, Nk, d,
                            causal, sc, rb, dt, P(w, 5), nb, S(strm))
    assert r in CODES
    r = lib.attn_prefill_cached(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), B, Hq, Hkv, Nq, Nk,
                                d, sc, rb, dt, causal, S(strm))
    assert r in CODES
    assert lib.attn_fwd_workspace_bytes(B, Hkv, Nk, d, rb, dt) == fwd_ws(B, Hkv, Nk, d, rb, dt)


@SETTINGS
@given(st.tuples(small, small, small, size, size, dims, flag, scale, base, dtype, ptr, wsb, ptr))
def test_bwd(a):
    B, Hq, Hkv, Nq, Nk, d, causal, sc, rb, dt, p, nb, w = a
    Nk = cap(Nk, rb)
    lib = L()
    r = lib.attn_bwd(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), P(p, 5), P(p, 6), P(p, 7),
                     P(p, 8), B, Hq, Hkv, Nq, Nk, d, causal, sc, rb, dt, P(w, 9), nb, None)
    assert r in CODES
    assert (lib.attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, rb, dt)
            == bwd_ws(B, Hq, Hkv, Nq, Nk, d, rb, dt))


@SETTINGS
@given(st.tuples(small, small, small, size, dims, scale, dtype, ptr, wsb, ptr))
def test_decode(a):
    B, Hq, Hkv, max_len, d, sc, dt, p, nb, w = a
    lib = L()
    r = lib.attn_decode(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), P(p, 5), B, Hq, Hkv, max_len,
                        d, sc, dt, P(w, 6), nb, None)
    assert r in CODES
    r = lib.attn_decode_noalloc(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), P(p, 5), B, Hq, Hkv,
                                max_len, d, sc, dt, None)
    assert r in CODES
    assert (lib.attn_decode_workspace_bytes(B, Hq, Hkv, max_len, d)
            == dec_ws(B, Hq, Hkv, 1, max_len, d, CHUNK))


@SETTINGS
@given(st.tuples(small, small, small, small, size, dims, scale, base, dtype, dtype, ptr, wsb, ptr))
def test_decode_multi(a):
    B, Hq, Hkv, T, max_len, d, sc, rb, dt, odt, p, nb, w = a
    max_len = cap(max_len, rb)
    lib = L()
    r = lib.attn_decode_multi(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), P(p, 5), B, Hq, Hkv, T,
                              max_len, d, sc, rb, dt, odt, P(w, 6), nb, None)
    assert r in CODES
    assert (lib.attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, max_len, d)
            == dec_ws(B, Hq, Hkv, T, max_len, d, CHUNK))


@SETTINGS
@given(st.tuples(small, small, small, small, size, size, size, dims, scale, base, dtype, dtype,
                 ptr, wsb, ptr))
def test_decode_paged(a):
    B, Hq, Hkv, T, max_blocks, block, nblocks, d, sc, rb, dt, odt, p, nb, w = a
    if rope_ok(rb) and max_blocks > 0 and block > 0:
        max_blocks = min(max_blocks, max(1, MAXPOS // block))
    lib = L()
    r = lib.attn_decode_paged(P(p, 0), P(p, 1), P(p, 2), P(p, 3), P(p, 4), P(p, 5), P(p, 6), B, Hq,
                              Hkv, T, nblocks, block, max_blocks, d, sc, rb, dt, odt, P(w, 7), nb,
                              None)
    assert r in CODES
    max_len = max_blocks * block if max_blocks > 0 and block > 0 else 0
    want = dec_ws(B, Hq, Hkv, T, max_len, d, CHUNK_PAGED) if max_len < (1 << 31) else 0
    assert lib.attn_decode_paged_workspace_bytes(B, Hq, Hkv, T, max_blocks, block, d) == want


@SETTINGS
@given(st.tuples(small, small, size, dims, size, base, dtype, ptr, ptr))
def test_rope_apply(a):
    B, H, N, d, off, rb, dt, p, strm = a
    if rope_ok(rb):
        N, off = min(N, MAXPOS), min(off, MAXPOS)
    lib = L()
    r = lib.attn_rope_apply(P(p, 0), P(p, 1), B, H, N, d, off, rb, dt, S(strm))
    assert r in CODES


def test_status_strings():
    lib = L()
    for c in range(-3, 8):
        assert lib.attn_status_str(c)
