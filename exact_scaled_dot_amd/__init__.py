"""Exact scaled-dot-product attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libattn.so`` (C ABI declared in ``include/attn.h``).
This module only marshals arguments: shapes, dtypes and pointers of torch
device tensors go to the library, which validates them and runs every step on
the GPU.  torch provides device memory and the current stream.  There is no
fallback: if the library is missing, every call raises.

Functions (same names as the C entry points):
  fwd(q, k, v, causal, scale=None, rope_base=0.0, out=None, lse=None, workspace=None,
      window=0)       (window > 0: attn_fwd_window, causal sliding window)
  bwd(q, k, v, o, lse, dout, causal, scale=None, rope_base=0.0, workspace=None)
  decode(q, k_cache, v_cache, seq_lens, scale=None, out=None, lse=None, workspace=None)
  decode_noalloc(q, k_cache, v_cache, seq_lens, scale=None, out=None, lse=None)
                      (no workspace: the library's static per-device array)
  decode_multi(q, k_cache, v_cache, seq_lens, scale=None, rope_base=0.0, out=None, lse=None,
               workspace=None)   (q [B,Hq,T,d]: T new tokens per sequence)
  decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale=None, rope_base=0.0, out=None,
               lse=None, workspace=None)   (pools [num_blocks, Hkv, block_size, d])
  prefill_cached(q, k_cache, v_cache, scale=None, rope_base=0.0, out=None, lse=None)
                      (chunked prefill over a cache with keys stored rotated)
  decode_multi, decode_paged and prefill_cached take out_dtype=torch.bfloat16 for a bf16 O
  rope_apply(x, rope_base, pos_offset=0, out=None)
  fwd_workspace_bytes(...), decode_workspace_bytes(...), decode_multi_workspace_bytes(...),
  decode_paged_workspace_bytes(...), status_str(code)
"""

from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_BF16 = 0
ATTN_F32 = 1
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_HIP",
          4: "ATTN_ERR_WORKSPACE"}

EXPORTS = ("attn_status_str", "attn_fwd_workspace_bytes", "attn_fwd", "attn_fwd_window",
           "attn_bwd_workspace_bytes", "attn_bwd",
           "attn_decode_workspace_bytes", "attn_decode", "attn_decode_multi_workspace_bytes",
           "attn_decode_multi", "attn_decode_paged_workspace_bytes", "attn_decode_paged",
           "attn_rope_apply", "attn_decode_noalloc", "attn_prefill_cached")

_lib = None


class AttnError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")


def lib():
    """Load libattn.so once; raise if it has not been built.

    torch is imported first.  torch ships its own HIP runtime and asks for it
    by the unversioned name, so if libattn.so (which asks for the versioned
    name of the system runtime) were loaded first, the process would hold two
    runtimes and torch's streams and device memory would be foreign to the
    library's.  Loaded after torch, libattn.so binds to torch's runtime."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_scaled_dot_amd.build`")
    import torch  # noqa: F401  (see above: one HIP runtime in the process)
    _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _declare(L):
    """Set the argument and result types of every entry point on a loaded
    library object (the C declarations of include/attn.h)."""
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_status_str.argtypes = [i]
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_fwd_workspace_bytes.argtypes = [i, i, i, i, f, i]
    L.attn_fwd_workspace_bytes.restype = sz
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, i, vp, sz, vp]
    L.attn_fwd.restype = i
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, i, vp, sz, vp]
    L.attn_fwd_window.restype = i
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i, f, i]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, i, vp,
                           sz, vp]
    L.attn_bwd.restype = i
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_decode.restype = i
    L.attn_decode_multi_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.attn_decode_multi_workspace_bytes.restype = sz
    L.attn_prefill_cached.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, i, i, vp]
    L.attn_prefill_cached.restype = i
    L.attn_decode_multi.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, i, i, vp, sz,
                                    vp]
    L.attn_decode_multi.restype = i
    L.attn_decode_paged_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_decode_paged_workspace_bytes.restype = sz
    L.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, f, i,
                                    i, vp, sz, vp]
    L.attn_decode_paged.restype = i
    L.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_decode_noalloc.restype = i
    L.attn_rope_apply.argtypes = [vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_rope_apply.restype = i
    return L


def status_str(code: int) -> str:
    return lib().attn_status_str(int(code)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(fn, code):
    if code != 0:
        raise AttnError(fn, code)


def _need_cuda_contig(name, t):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    # kernels run on the current device and its current stream
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, but the current device is "
                         f"cuda:{torch.cuda.current_device()}")


def _check_out(name, t, shape, dtype):
    """A caller-supplied output or workspace: the kernels write exactly `shape`
    elements of `dtype` from its first element, so anything else is rejected."""
    if t is None:
        return
    _need_cuda_contig(name, t)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _out_code(dtype) -> int:
    """Output dtype code: torch.float32 -> ATTN_F32, torch.bfloat16 -> ATTN_BF16."""
    import torch
    if dtype == torch.float32:
        return ATTN_F32
    if dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"output dtype must be float32 or bfloat16, got {dtype}")


def fwd_workspace_bytes(B, Hkv, Nk, d, rope_base, dtype_code) -> int:
    return int(lib().attn_fwd_workspace_bytes(B, Hkv, Nk, d, float(rope_base), dtype_code))


def decode_workspace_bytes(B, Hq, Hkv, max_len, d) -> int:
    return int(lib().attn_decode_workspace_bytes(B, Hq, Hkv, max_len, d))


def decode_multi_workspace_bytes(B, Hq, Hkv, T, max_len, d) -> int:
    return int(lib().attn_decode_multi_workspace_bytes(B, Hq, Hkv, T, max_len, d))


def fwd(q, k, v, causal: bool, scale=None, rope_base: float = 0.0, out=None, lse=None,
        workspace=None, want_lse: bool = True, window: int = 0):
    """O [B,Hq,Nq,d] fp32 and lse [B,Hq,Nq] fp32 of softmax(scale QK^T + M) V.

    window > 0 selects the causal sliding window (attn_fwd_window; causal must
    then be true): the query at position p sees keys p-window+1 .. p."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_cuda_contig(n, t)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("shape mismatch between q, k and v")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_out("out", out, (B, Hq, Nq, d), torch.float32)
    _check_out("lse", lse, (B, Hq, Nq), torch.float32)
    _check_out("workspace", workspace, None, torch.uint8)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    need = fwd_workspace_bytes(B, Hkv, Nk, d, rope_base, code)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if window:
        if not causal:
            raise ValueError("the sliding window is causal: pass causal=True")
        _check("attn_fwd_window", L.attn_fwd_window(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, int(window),
            float(scale), float(rope_base), code, _ptr(workspace), wsb, _stream()))
        return out, lse
    _check("attn_fwd", L.attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv,
                                  Nq, Nk, d, int(bool(causal)), float(scale), float(rope_base),
                                  code, _ptr(workspace), wsb, _stream()))
    return out, lse


def prefill_cached(q, k_cache, v_cache, scale=None, rope_base: float = 0.0, out=None, lse=None,
                   out_dtype=None, want_lse: bool = True):
    """Chunked prefill (attn_prefill_cached): q [B,Hq,Nq,d] are the last Nq
    positions of caches k_cache, v_cache [B,Hkv,Nk,d] whose keys are stored
    already rotated; query i sits at Nk - Nq + i and sees keys up to there.
    O is float32, or bfloat16 with out_dtype=torch.bfloat16."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need_cuda_contig(n, t)
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, k_cache, v_cache must share a dtype")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k_cache.shape
    if (Bk, dk) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch between q and the caches")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    _check_out("out", out, (B, Hq, Nq, d), out_dtype)
    _check_out("lse", lse, (B, Hq, Nq), torch.float32)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check("attn_prefill_cached", L.attn_prefill_cached(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
        float(scale), float(rope_base), _dtype_code(q), _out_code(out_dtype), _stream()))
    return out, lse


def bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, rope_base, dtype_code) -> int:
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, float(rope_base), dtype_code))


def bwd(q, k, v, o, lse, dout, causal: bool, scale=None, rope_base: float = 0.0, dq=None,
        dk=None, dv=None, workspace=None):
    """dq [B,Hq,Nq,d], dk, dv [B,Hkv,Nk,d] (fp32) of sum(dout * O) for O = fwd(q, k, v)."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        _need_cuda_contig(n, t)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if o.dtype != torch.float32 or lse.dtype != torch.float32 or dout.dtype != torch.float32:
        raise TypeError("o, lse and dout must be float32")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if ((Bk, dk_) != (B, d) or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape)
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq)):
        raise ValueError("shape mismatch between q, k, v, o, lse and dout")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_out("dq", dq, (B, Hq, Nq, d), torch.float32)
    _check_out("dk", dk, (B, Hkv, Nk, d), torch.float32)
    _check_out("dv", dv, (B, Hkv, Nk, d), torch.float32)
    _check_out("workspace", workspace, None, torch.uint8)
    if dq is None:
        dq = torch.empty((B, Hq, Nq, d), dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty((B, Hkv, Nk, d), dtype=torch.float32, device=q.device)
    need = bwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, rope_base, code)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("attn_bwd", L.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                  _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Nq, Nk, d,
                                  int(bool(causal)), float(scale), float(rope_base), code,
                                  _ptr(workspace), wsb, _stream()))
    return dq, dk, dv


def decode(q, k_cache, v_cache, seq_lens, scale=None, out=None, lse=None, workspace=None,
           want_lse: bool = True):
    """One-query attention per sequence over cache rows 0..seq_lens[b]-1."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        _need_cuda_contig(n, t)
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    B, Hq, d = q.shape
    Bc, Hkv, max_len, dc = k_cache.shape
    if (Bc, dc) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape) or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_out("out", out, (B, Hq, d), torch.float32)
    _check_out("lse", lse, (B, Hq), torch.float32)
    _check_out("workspace", workspace, None, torch.uint8)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(B, Hq, Hkv, max_len, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("attn_decode", L.attn_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens),
                                        _ptr(out), _ptr(lse), B, Hq, Hkv, max_len, d,
                                        float(scale), code, _ptr(workspace), wsb, _stream()))
    return out, lse


# Capacity of the library's static per-device array (ATTN_DECODE_NOALLOC_MAX_BYTES).
DECODE_NOALLOC_MAX_BYTES = 16 << 20


def decode_noalloc(q, k_cache, v_cache, seq_lens, scale=None, out=None, lse=None):
    """``decode`` without a workspace (attn_decode_noalloc): the partial states
    live in the library's static per-device array, so with ``out`` and ``lse``
    given the call allocates nothing.  Calls that overlap on one device race."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        _need_cuda_contig(n, t)
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    B, Hq, d = q.shape
    Bc, Hkv, max_len, dc = k_cache.shape
    if (Bc, dc) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape) or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_out("out", out, (B, Hq, d), torch.float32)
    _check_out("lse", lse, (B, Hq), torch.float32)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _check("attn_decode_noalloc", L.attn_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv,
        max_len, d, float(scale), _dtype_code(q), _stream()))
    return out, lse


def decode_multi(q, k_cache, v_cache, seq_lens, scale=None, rope_base: float = 0.0, out=None,
                 lse=None, workspace=None, want_lse: bool = True, out_dtype=None):
    """T new tokens per sequence (q [B,Hq,T,d]); token t of sequence b sits at
    position seq_lens[b] - T + t and sees cache rows up to that position.  O is
    float32, or bfloat16 with out_dtype=torch.bfloat16."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        _need_cuda_contig(n, t)
    if seq_lens.dtype != torch.int32:
        raise TypeError("seq_lens must be int32")
    B, Hq, T, d = q.shape
    Bc, Hkv, max_len, dc = k_cache.shape
    if (Bc, dc) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape) or seq_lens.numel() != B:
        raise ValueError("shape mismatch between q, caches and seq_lens")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    _check_out("out", out, (B, Hq, T, d), out_dtype)
    _check_out("lse", lse, (B, Hq, T), torch.float32)
    _check_out("workspace", workspace, None, torch.uint8)
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    need = decode_multi_workspace_bytes(B, Hq, Hkv, T, max_len, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("attn_decode_multi", L.attn_decode_multi(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_lens), _ptr(out), _ptr(lse), B, Hq, Hkv,
        T, max_len, d, float(scale), float(rope_base), code, _out_code(out_dtype), _ptr(workspace),
        wsb, _stream()))
    return out, lse


def decode_paged_workspace_bytes(B, Hq, Hkv, T, max_blocks, block_size, d) -> int:
    return int(lib().attn_decode_paged_workspace_bytes(B, Hq, Hkv, T, max_blocks, block_size, d))


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale=None, rope_base: float = 0.0,
                 out=None, lse=None, workspace=None, want_lse: bool = True, out_dtype=None):
    """decode_multi over a paged cache: token p of sequence b is row p % block_size
    of pool block block_table[b, p // block_size]."""
    import torch
    L = lib()
    for n, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("block_table", block_table),
                 ("seq_lens", seq_lens)):
        _need_cuda_contig(n, t)
    if seq_lens.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise TypeError("seq_lens and block_table must be int32")
    B, Hq, T, d = q.shape
    num_blocks, Hkv, block_size, dp = k_pool.shape
    Bt, max_blocks = block_table.shape
    if (dp != d or tuple(v_pool.shape) != tuple(k_pool.shape) or seq_lens.numel() != B
            or Bt != B):
        raise ValueError("shape mismatch between q, pools, block_table and seq_lens")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype is None:
        out_dtype = torch.float32 if out is None else out.dtype
    _check_out("out", out, (B, Hq, T, d), out_dtype)
    _check_out("lse", lse, (B, Hq, T), torch.float32)
    _check_out("workspace", workspace, None, torch.uint8)
    if out is None:
        out = torch.empty((B, Hq, T, d), dtype=out_dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    need = decode_paged_workspace_bytes(B, Hq, Hkv, T, max_blocks, block_size, d)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("attn_decode_paged", L.attn_decode_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(block_table), _ptr(seq_lens), _ptr(out),
        _ptr(lse), B, Hq, Hkv, T, num_blocks, block_size, max_blocks, d, float(scale),
        float(rope_base), code, _out_code(out_dtype), _ptr(workspace), wsb, _stream()))
    return out, lse


def rope_apply(x, rope_base: float, pos_offset: int = 0, out=None):
    """RoPE of x [B,H,N,d] at positions pos_offset + n, rounded to x's dtype."""
    import torch
    L = lib()
    _need_cuda_contig("x", x)
    B, H, N, d = x.shape
    _check_out("out", out, (B, H, N, d), x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _check("attn_rope_apply", L.attn_rope_apply(_ptr(x), _ptr(out), B, H, N, d, int(pos_offset),
                                                float(rope_base), _dtype_code(x), _stream()))
    return out
