"""Python binding of libmiattn (exact attention on one MI355X).

Argument marshalling only: tensors supply device pointers, sizes and the
current HIP stream; every step of the computation runs in the library's HIP
kernels. The library is loaded from this package directory; if it is missing
the import of any entry point raises (there is no fallback implementation).

Layouts: q, o, dout, dq [B, N, H, d]; k, v, dk, dv [B, N, Hkv, d];
lse [B, H, N] float32. Supported: d in {64, 128}; dtype float32 or bfloat16.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["fwd", "bwd", "bwd_noalloc", "merge", "fwd_chunked", "bwd_chunked", "fwd_kvcache", "fwd_varlen", "bwd_varlen",
           "fwd_blocksparse", "bwd_blocksparse", "block_mask_shape",
           "release_scratch", "lib", "MiattnError",
           "library_path", "balanced_rounds"]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmiattn.so")

F32, BF16 = 0, 1
_STATUS = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "ELAUNCH", 4: "ENOMEM"}


class MiattnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("libmiattn %s: %s" % (_STATUS.get(code, code), msg))
        self.code = code


_lib = None


def lib():
    """The loaded libmiattn (ctypes.CDLL). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError("libmiattn.so is not built (expected at %s); run "
                          "`python -m exact_attention_37_amd.build`" % library_path)
    L = ctypes.CDLL(library_path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i]
    L.attn_bwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i]
    L.attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i]
    L.attn_bwd_timed.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i, vp]
    L.attn_fwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i]
    L.attn_bwd_window.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i]
    L.attn_merge.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp]
    L.attn_fwd_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, i]
    L.attn_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, i]
    L.attn_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i]
    L.attn_fwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, i]
    L.attn_bwd_blocksparse.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i]
    L.attn_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, i]
    L.attn_bwd_chunked.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, vp, vp, vp, i, i]
    for fn in ("attn_fwd", "attn_bwd", "attn_bwd_noalloc", "attn_bwd_timed", "attn_merge", "attn_fwd_chunked", "attn_bwd_chunked",
               "attn_fwd_kvcache", "attn_fwd_window", "attn_bwd_window", "attn_fwd_varlen", "attn_bwd_varlen",
               "attn_fwd_blocksparse", "attn_bwd_blocksparse"):
        getattr(L, fn).restype = i
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_last_error.argtypes = []
    L.attn_version.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_release_scratch.argtypes = [vp]
    L.attn_release_scratch.restype = i
    ip = ctypes.POINTER(ctypes.c_int)
    L.attn_chunk_schedule.argtypes = [i, ip, ip, ip, i]
    L.attn_chunk_schedule.restype = i
    _lib = L
    return L


def _check(status):
    if status != 0:
        raise MiattnError(status, lib().attn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s" % (name, device))


def _dims(q, k, v):
    _need(q, "q")
    dt = q.dtype
    _dtype_code(q)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, N, heads, d]")
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    _need(k, "k", dt, (B, N, Hkv, d), q.device)
    _need(v, "v", dt, (B, N, Hkv, d), q.device)
    return B, N, H, Hkv, d


def fwd(q, k, v, causal=False, scale=None, out=None, out_lse=None, window=0):
    """Exact attention forward. Returns (o, lse).

    window > 0: causal sliding-window attention (attn_fwd_window): query row
    i sees key rows i - window < j <= i; causal is implied.
    """
    B, N, H, Hkv, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if out_lse is None else out_lse
    _need(o, "out", q.dtype, q.shape, q.device)
    _need(lse, "out_lse", torch.float32, (B, H, N), q.device)
    if window:
        _check(lib().attn_fwd_window(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                     int(window), scale, _stream(q), _dtype_code(q)))
    else:
        _check(lib().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                              int(bool(causal)), scale, _stream(q), _dtype_code(q)))
    return o, lse


def bwd(q, k, v, o, lse, dout, causal=False, scale=None, accumulate=False, dq=None, dk=None, dv=None,
        marks=None, window=0):
    """Exact attention backward from the forward's o and lse. Returns (dq, dk, dv).

    accumulate=True: dq/dk/dv are float32 tensors (given or zero-initialised)
    that the gradients are added to; otherwise they have q's dtype.
    marks: optional pair of torch.cuda.Event, recorded on the stream after the
    backward's first and second kernel (attn_bwd_timed): for bf16 the dQ
    kernel (which also forms the rowsum of dout * o) and the dK/dV kernel.
    window > 0: backward of causal sliding-window attention (attn_bwd_window).
    """
    B, N, H, Hkv, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _need(o, "o", q.dtype, q.shape, q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    gdt = torch.float32 if accumulate else q.dtype
    mk = (lambda t: torch.zeros(t.shape, dtype=gdt, device=q.device)) if accumulate else \
         (lambda t: torch.empty(t.shape, dtype=gdt, device=q.device))
    dq = mk(q) if dq is None else dq
    dk = mk(k) if dk is None else dk
    dv = mk(v) if dv is None else dv
    _need(dq, "dq", gdt, q.shape, q.device)
    _need(dk, "dk", gdt, k.shape, q.device)
    _need(dv, "dv", gdt, v.shape, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d, int(bool(causal)), scale,
            _stream(q), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(q), int(bool(accumulate)))
    if window:
        if marks is not None:
            raise ValueError("marks are not supported with a window")
        wargs = args[:10] + (int(window),) + args[11:]
        _check(lib().attn_bwd_window(*wargs))
    elif marks is None:
        _check(lib().attn_bwd(*args))
    else:
        for m in marks:           # torch creates the HIP event at its first record
            if not m.cuda_event:
                m.record()
        ev = (ctypes.c_void_p * 2)(*[ctypes.c_void_p(m.cuda_event) for m in marks])
        _check(lib().attn_bwd_timed(*args, ev))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dout, causal, scale, dq, dk, dv, accumulate=False):
    """attn_bwd_noalloc: the backward into caller-given dq, dk, dv with the
    library's fixed per-device rowsum array, allocating nothing (B * H * N at
    most 4194304). Returns (dq, dk, dv)."""
    B, N, H, Hkv, d = _dims(q, k, v)
    _need(o, "o", q.dtype, q.shape, q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    gdt = torch.float32 if accumulate else q.dtype
    _need(dq, "dq", gdt, q.shape, q.device)
    _need(dk, "dk", gdt, k.shape, q.device)
    _need(dv, "dv", gdt, v.shape, q.device)
    _check(lib().attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                  int(bool(causal)), float(scale), _stream(q), _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _dtype_code(q), int(bool(accumulate))))
    return dq, dk, dv


def merge(o_a, lse_a, o_b, lse_b, out=None, out_lse=None):
    """LSE merge of partials over disjoint key sets. Returns (o, lse).

    out/out_lse may be o_a/lse_a (or o_b/lse_b) for an in-place merge."""
    _need(o_a, "o_a")
    B, N, H, d = o_a.shape
    _need(o_b, "o_b", o_a.dtype, o_a.shape, o_a.device)
    _need(lse_a, "lse_a", torch.float32, (B, H, N), o_a.device)
    _need(lse_b, "lse_b", torch.float32, (B, H, N), o_a.device)
    o = torch.empty_like(o_a) if out is None else out
    lse = torch.empty_like(lse_a) if out_lse is None else out_lse
    _need(o, "out", o_a.dtype, o_a.shape, o_a.device)
    _need(lse, "out_lse", torch.float32, (B, H, N), o_a.device)
    _check(lib().attn_merge(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse),
                            B, H, N, d, _dtype_code(o_a), _stream(o_a)))
    return o, lse


def fwd_chunked(q, k, v, nchunks, scale=None):
    """Causal forward as balanced rounds of chunk pairs merged by LSE. Returns (o, lse)."""
    B, N, H, Hkv, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check(lib().attn_fwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                  scale, _stream(q), _dtype_code(q), int(nchunks)))
    return o, lse


def bwd_chunked(q, k, v, o, lse, dout, nchunks, scale=None):
    """Causal backward over the same chunk pairs, float32 accumulation. Returns (dq, dk, dv)."""
    B, N, H, Hkv, d = _dims(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _need(o, "o", q.dtype, q.shape, q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _check(lib().attn_bwd_chunked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, N, d,
                                  scale, _stream(q), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                  _dtype_code(q), int(nchunks)))
    return dq, dk, dv


def fwd_kvcache(q, k_cache, v_cache, k_lens=None, causal=True, scale=None, nsplit=0, out=None, out_lse=None):
    """Nq new query rows against a key/value cache (attn_fwd_kvcache, bf16).

    q: [B, Nq, H, d]; k_cache, v_cache: [B, Nk, Hkv, d]; k_lens: int32 tensor
    [B] of valid cache rows on the same device, or None for Nk. Under causal,
    query row i of batch b sits at position k_lens[b] - Nq + i. nsplit = 0
    lets the library choose the number of key chunks. Returns (o, lse) with
    lse [B, H, Nq] float32.
    """
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q and the caches must be 4-D [B, rows, heads, d]")
    B, Nq, H, d = q.shape
    Nk, Hkv = k_cache.shape[1], k_cache.shape[2]
    _need(k_cache, "k_cache", torch.bfloat16, (B, Nk, Hkv, d), q.device)
    _need(v_cache, "v_cache", torch.bfloat16, (B, Nk, Hkv, d), q.device)
    if k_lens is not None:
        _need(k_lens, "k_lens", torch.int32, (B,), q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if out_lse is None else out_lse
    _need(o, "out", q.dtype, q.shape, q.device)
    _need(lse, "out_lse", torch.float32, (B, H, Nq), q.device)
    _check(lib().attn_fwd_kvcache(_ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  None if k_lens is None else _ptr(k_lens), _ptr(o), _ptr(lse),
                                  B, H, Hkv, Nq, Nk, d, int(bool(causal)), scale, int(nsplit),
                                  _stream(q), _dtype_code(q)))
    return o, lse


def _varlen_dims(q, k, v, cu_seqlens, max_len):
    _need(q, "q")
    dt = q.dtype
    _dtype_code(q)
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed q, k, v must be 3-D [total, heads, d]")
    total, H, d = q.shape
    Hkv = k.shape[1]
    _need(k, "k", dt, (total, Hkv, d), q.device)
    _need(v, "v", dt, (total, Hkv, d), q.device)
    _need(cu_seqlens, "cu_seqlens", torch.int32, None, q.device)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be 1-D with nseq + 1 >= 2 entries")
    return cu_seqlens.numel() - 1, int(max_len), total, H, Hkv, d


def fwd_varlen(q, k, v, cu_seqlens, max_len, causal=False, scale=None, window=0, out=None, out_lse=None):
    """Forward over a packed batch of sequences of different lengths (attn_fwd_varlen).

    q: [total, H, d]; k, v: [total, Hkv, d]; cu_seqlens: int32 device tensor
    [nseq + 1] of row offsets (0, ..., total); max_len: the longest sequence.
    Each sequence attends only within itself. Returns (o, lse), lse [H, total].
    """
    nseq, max_len, total, H, Hkv, d = _varlen_dims(q, k, v, cu_seqlens, max_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, total), dtype=torch.float32, device=q.device) if out_lse is None else out_lse
    _need(o, "out", q.dtype, q.shape, q.device)
    _need(lse, "out_lse", torch.float32, (H, total), q.device)
    _check(lib().attn_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), nseq,
                                 max_len, total, H, Hkv, d, int(bool(causal)), int(window), scale,
                                 _stream(q), _dtype_code(q)))
    return o, lse


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_len, causal=False, scale=None, window=0,
               accumulate=False, dq=None, dk=None, dv=None):
    """Backward of fwd_varlen from its o and lse (attn_bwd_varlen). Returns (dq, dk, dv)."""
    nseq, max_len, total, H, Hkv, d = _varlen_dims(q, k, v, cu_seqlens, max_len)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _need(o, "o", q.dtype, q.shape, q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, (H, total), q.device)
    gdt = torch.float32 if accumulate else q.dtype
    mk = (lambda t: torch.zeros(t.shape, dtype=gdt, device=q.device)) if accumulate else \
         (lambda t: torch.empty(t.shape, dtype=gdt, device=q.device))
    dq = mk(q) if dq is None else dq
    dk = mk(k) if dk is None else dk
    dv = mk(v) if dv is None else dv
    _need(dq, "dq", gdt, q.shape, q.device)
    _need(dk, "dk", gdt, k.shape, q.device)
    _need(dv, "dv", gdt, v.shape, q.device)
    _check(lib().attn_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_seqlens), nseq,
                                 max_len, total, H, Hkv, d, int(bool(causal)), int(window), scale,
                                 _stream(q), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(q),
                                 int(bool(accumulate))))
    return dq, dk, dv


BLOCK_ROWS, BLOCK_COLS = 256, 128


def block_mask_shape(N):
    """Shape of the block mask for sequence length N: one entry per block of
    BLOCK_ROWS query rows x BLOCK_COLS keys."""
    return ((N + BLOCK_ROWS - 1) // BLOCK_ROWS, (N + BLOCK_COLS - 1) // BLOCK_COLS)


def _block_mask(block_mask, N, device):
    _need(block_mask, "block_mask", torch.uint8, block_mask_shape(N), device)
    return block_mask


def fwd_blocksparse(q, k, v, block_mask, causal=False, scale=None, out=None, out_lse=None):
    """Block-sparse attention forward (attn_fwd_blocksparse). block_mask: uint8
    device tensor of block_mask_shape(N); a zero entry removes its block of
    query rows x keys. Returns (o, lse); rows with no key get o = 0, lse = -inf."""
    B, N, H, Hkv, d = _dims(q, k, v)
    _block_mask(block_mask, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if out_lse is None else out_lse
    _need(o, "out", q.dtype, q.shape, q.device)
    _need(lse, "out_lse", torch.float32, (B, H, N), q.device)
    _check(lib().attn_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(block_mask), B, H, Hkv,
                                      N, d, int(bool(causal)), scale, _stream(q), _dtype_code(q)))
    return o, lse


def bwd_blocksparse(q, k, v, o, lse, dout, block_mask, causal=False, scale=None, accumulate=False,
                    dq=None, dk=None, dv=None):
    """Backward of fwd_blocksparse with the same block_mask. Returns (dq, dk, dv)."""
    B, N, H, Hkv, d = _dims(q, k, v)
    _block_mask(block_mask, N, q.device)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    _need(o, "o", q.dtype, q.shape, q.device)
    _need(dout, "dout", q.dtype, q.shape, q.device)
    _need(lse, "lse", torch.float32, (B, H, N), q.device)
    gdt = torch.float32 if accumulate else q.dtype
    mk = (lambda t: torch.zeros(t.shape, dtype=gdt, device=q.device)) if accumulate else \
         (lambda t: torch.empty(t.shape, dtype=gdt, device=q.device))
    dq = mk(q) if dq is None else dq
    dk = mk(k) if dk is None else dk
    dv = mk(v) if dv is None else dv
    _need(dq, "dq", gdt, q.shape, q.device)
    _need(dk, "dk", gdt, k.shape, q.device)
    _need(dv, "dv", gdt, v.shape, q.device)
    _check(lib().attn_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(block_mask), B, H, Hkv,
                                      N, d, int(bool(causal)), scale, _stream(q), _ptr(dout), _ptr(dq), _ptr(dk),
                                      _ptr(dv), _dtype_code(q), int(bool(accumulate))))
    return dq, dk, dv


def release_scratch(stream=None):
    """Frees the scratch buffer the library keeps for `stream` (a
    torch.cuda.Stream, default the current stream) on the current device, in
    stream order (attn_release_scratch)."""
    s = torch.cuda.current_stream() if stream is None else stream
    _check(lib().attn_release_scratch(ctypes.c_void_p(s.cuda_stream)))


def balanced_rounds(P):
    """The library's chunk-pair schedule for P chunks: a list of rounds, each a
    list of (query chunk, key chunk) pairs in processing order."""
    n = P * (P + 1) // 2
    arr = ctypes.c_int * max(n, 1)
    r, qc, kc = arr(), arr(), arr()
    got = lib().attn_chunk_schedule(int(P), r, qc, kc, n)
    if got < 0:
        raise ValueError("invalid chunk count %r" % P)
    rounds = []
    for t in range(got):
        if r[t] == len(rounds):
            rounds.append([])
        rounds[r[t]].append((qc[t], kc[t]))
    return rounds
