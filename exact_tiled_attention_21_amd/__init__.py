"""Exact tiled attention for MI355X: the Python face of libfa (include/fa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libfa.so. torch supplies device memory and the current stream.

  attention(q, k, v, causal=False, scale=None) -> (o, lse)
  attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                   causal=False, scale=None) -> (o, lse)
  decode(q, k_cache, v_cache, num_splits=16, scale=None, causal=False) -> (o, lse)
  decode_noalloc(q, k_cache, v_cache, num_splits=16, scale=None, causal=False,
                 out=None, lse=None) -> (o, lse)
  decode_paged(q, k_pages, v_pages, block_table, cache_seqlens, num_splits=16,
               scale=None, causal=False) -> (o, lse)
  attention_backward(q, k, v, o, lse, dout, causal=False, scale=None,
                     window=(-1, -1)) -> (dq, dk, dv)
  attention_varlen_backward(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k,
                            max_seqlen_q, max_seqlen_k, causal=False, scale=None) -> (dq, dk, dv)
  attention_func(q, k, v, causal=False, scale=None, window=(-1, -1)) -> o, differentiable

Tensors are [batch, seq_len, heads, head_dim], fp16 or bf16, contiguous, on a
ROCm device; lse is float32 [batch, heads, seq_len_q]. The default scale is
1/sqrt(head_dim) ("flash-attention-v100" README, How to use FlashAttention).
"""
from __future__ import annotations

import ctypes
import math

from ._lib import FA_BF16, FA_F16, FA_MAX_SPLITS, FA_NOALLOC_SCRATCH_BYTES, FaError, load, status_str  # noqa: F401

__all__ = ["attention", "attention_varlen", "attention_backward", "attention_varlen_backward", "attention_func",
           "bwd_workspace_bytes", "decode", "decode_noalloc",
           "decode_paged", "decode_workspace_bytes", "FaError", "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"dtype must be float16 or bfloat16, got {t.dtype}")


def _check(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [batch, seq_len, heads, head_dim]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("batch and head_dim of q and k must match")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")


def _check_given(name, t, shape, dtype, device):
    """A caller-supplied output must be exactly what the kernels write into: a smaller,
    strided or host tensor would let them write outside it."""
    if t is None:
        return
    if (not t.is_cuda or t.device != device or tuple(t.shape) != tuple(shape) or t.dtype != dtype
            or not t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")


def _check_on(name, t, device):
    if not t.is_cuda or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {device}")


def _stream(t):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
              window=(-1, -1)):
    """Exact attention forward: softmax(scale * q k^T [+ causal mask or sliding-window
    band]) v, plus per-row LSE. window = (left, right) keys around the bottom-right
    aligned diagonal, -1 for an open side."""
    torch = _torch()
    _check(q, k, v)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_given("out", out, q.shape, q.dtype, q.device)
    _check_given("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        if tuple(window) == (-1, -1):
            st = load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                               B, Nq, Nk, Hq, Hkv, d, int(bool(causal)), float(scale), _dtype_code(q),
                               _stream(q))
        else:
            st = load().fa_fwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse_t.data_ptr(), B, Nq, Nk, Hq, Hkv, d, int(window[0]),
                                      int(window[1]), int(bool(causal)), float(scale), _dtype_code(q),
                                      _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd")
    return o, lse_t


def decode_workspace_bytes(B: int, Nq: int, Hq: int, d: int, num_splits: int) -> int:
    return int(load().fa_decode_workspace_bytes(B, Nq, Hq, d, num_splits))


def decode(q, k_cache, v_cache, num_splits: int = 16, scale: float | None = None,
           causal: bool = False, workspace=None, out=None, lse=None):
    """Split-KV (Flash-Decoding) attention of a short query block over a KV cache."""
    torch = _torch()
    _check(q, k_cache, v_cache)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, Nq, Hq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_on("workspace", workspace, q.device)
    _check_given("out", out, q.shape, q.dtype, q.device)
    _check_given("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        st = load().fa_decode_splitkv(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(),
                                      lse_t.data_ptr(), B, Nq, Nk, Hq, Hkv, d, int(num_splits),
                                      int(bool(causal)), float(scale), _dtype_code(q),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(q))
    if st != 0:
        raise FaError(st, "fa_decode_splitkv")
    return o, lse_t


def decode_noalloc(q, k_cache, v_cache, num_splits: int = 16, scale: float | None = None,
                   causal: bool = False, out=None, lse=None):
    """decode() through fa_decode_splitkv_noalloc: the library takes the partials from
    a fixed device array instead of a workspace (calls that overlap on one GPU race
    on it). With out and lse given, nothing is allocated on this path."""
    torch = _torch()
    _check(q, k_cache, v_cache)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check_given("out", out, q.shape, q.dtype, q.device)
    _check_given("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        st = load().fa_decode_splitkv_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                              o.data_ptr(), lse_t.data_ptr(), B, Nq, Nk, Hq, Hkv, d,
                                              int(num_splits), int(bool(causal)), float(scale),
                                              _dtype_code(q), _stream(q))
    if st != 0:
        raise FaError(st, "fa_decode_splitkv_noalloc")
    return o, lse_t


def decode_paged(q, k_pages, v_pages, block_table, cache_seqlens, num_splits: int = 16,
                 scale: float | None = None, causal: bool = False, workspace=None, out=None, lse=None):
    """Split-KV attention over a paged KV cache.

    k_pages, v_pages: [num_pages, page_size, Hkv, d] page pools; block_table: int32
    [B, max_pages_per_seq] page indices per sequence; cache_seqlens: int32 [B] keys
    per sequence. page_size must be a multiple of 32."""
    torch = _torch()
    for name, t in (("q", q), ("k_pages", k_pages), ("v_pages", v_pages)):
        if not t.is_cuda or t.dim() != 4 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous 4-d device tensor")
    if not (q.dtype == k_pages.dtype == v_pages.dtype):
        raise TypeError("q, k_pages, v_pages must share a dtype")
    if k_pages.shape != v_pages.shape or q.shape[3] != k_pages.shape[3]:
        raise ValueError("k_pages and v_pages must match, and share head_dim with q")
    for name, t in (("block_table", block_table), ("cache_seqlens", cache_seqlens)):
        if not t.is_cuda or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    for name, t in (("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
                    ("cache_seqlens", cache_seqlens)):
        _check_on(name, t, q.device)
    B, Nq, Hq, d = q.shape
    num_pages, page_size, Hkv = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(cache_seqlens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages_per_seq] and cache_seqlens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = decode_workspace_bytes(B, Nq, Hq, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_on("workspace", workspace, q.device)
    _check_given("out", out, q.shape, q.dtype, q.device)
    _check_given("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        st = load().fa_decode_splitkv_paged(
            q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
            cache_seqlens.data_ptr(), o.data_ptr(), lse_t.data_ptr(), B, Nq, Hq, Hkv, d, num_pages,
            page_size, block_table.shape[1], int(num_splits), int(bool(causal)), float(scale),
            _dtype_code(q), workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise FaError(st, "fa_decode_splitkv_paged")
    return o, lse_t


def _check_max_seqlen(cu, max_seqlen, name):
    """Every sequence of the prefix sums `cu` is at most max_seqlen long (one
    device-to-host read of the prefix sums)."""
    longest = int((cu[1:] - cu[:-1]).max().item()) if cu.numel() > 1 else 0
    if longest > int(max_seqlen):
        raise ValueError(f"{name} = {max_seqlen} is below the longest sequence ({longest} rows)")


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                     scale: float | None = None, out=None, lse=None, validate: bool = True):
    """Exact attention over a packed batch of variable-length sequences.

    q [total_q, Hq, d], k/v [total_k, Hkv, d]; cu_seqlens_q/k int32 [B + 1] prefix
    sums on the device; returns o like q and lse float32 [Hq, total_q].
    max_seqlen_q must be at least every sequence's query count; validate=True
    checks that (one read of the prefix sums to the host), validate=False trusts
    the caller."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [tokens, heads, head_dim] device tensor")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share a dtype")
    if k.shape != v.shape or q.shape[2] != k.shape[2]:
        raise ValueError("k and v must match, and share head_dim with q")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device vector")
    if cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 entries")
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    for name, t in (("k", k), ("v", v), ("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _check_on(name, t, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if validate:
        _check_max_seqlen(cu_seqlens_q, max_seqlen_q, "max_seqlen_q")
    _check_given("out", out, q.shape, q.dtype, q.device)
    _check_given("lse", lse, (Hq, total_q), torch.float32, q.device)
    o = torch.empty_like(q) if out is None else out
    lse_t = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device) if lse is None else lse
    with torch.cuda.device(q.device):
        st = load().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse_t.data_ptr(),
                                  cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, int(max_seqlen_q),
                                  total_q, total_k, Hq, Hkv, d, int(bool(causal)), float(scale),
                                  _dtype_code(q), _stream(q))
    if st != 0:
        raise FaError(st, "fa_fwd_varlen")
    return o, lse_t


def bwd_workspace_bytes(B: int, Nq: int, Hq: int) -> int:
    return int(load().fa_bwd_workspace_bytes(B, Nq, Hq))


def attention_backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
                       workspace=None, dq=None, dk=None, dv=None, window=(-1, -1)):
    """Gradients (dq, dk, dv) of attention(q, k, v, causal, scale, window=window) for the
    upstream gradient dout, from the forward's output o and lse (float32 [B, Hq, Nq])."""
    torch = _torch()
    _check(q, k, v)
    for name, t in (("o", o), ("dout", dout)):
        _check_given(name, t, q.shape, q.dtype, q.device)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    _check_given("lse", lse, (B, Hq, Nq), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = bwd_workspace_bytes(B, Nq, Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_on("workspace", workspace, q.device)
    _check_given("dq", dq, q.shape, q.dtype, q.device)
    _check_given("dk", dk, k.shape, k.dtype, q.device)
    _check_given("dv", dv, v.shape, v.dtype, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    with torch.cuda.device(q.device):
        if tuple(window) == (-1, -1):
            st = load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Nq, Nk, Hq, Hkv,
                               d, int(bool(causal)), float(scale), _dtype_code(q), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(q))
        else:
            st = load().fa_bwd_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                      dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, Nq, Nk,
                                      Hq, Hkv, d, int(window[0]), int(window[1]), int(bool(causal)),
                                      float(scale), _dtype_code(q), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def attention_varlen_backward(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int,
                              max_seqlen_k: int, causal: bool = False, scale: float | None = None,
                              workspace=None, dq=None, dk=None, dv=None, validate: bool = True):
    """Gradients of attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, ...) for dout.

    q, o, dout [total_q, Hq, d]; k, v [total_k, Hkv, d]; lse float32 [Hq, total_q] as
    attention_varlen returns it; max_seqlen_q/k at least every sequence's length
    (validate=True checks that with one read of the prefix sums to the host)."""
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        if not t.is_cuda or t.dim() != 3 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous [tokens, heads, head_dim] device tensor")
    if not (q.dtype == k.dtype == v.dtype == o.dtype == dout.dtype):
        raise TypeError("q, k, v, o, dout must share a dtype")
    if k.shape != v.shape or q.shape[2] != k.shape[2] or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k and v must match; o and dout must match q; head_dim must agree")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device vector")
    if cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have B + 1 entries")
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("cu_seqlens_q", cu_seqlens_q),
                    ("cu_seqlens_k", cu_seqlens_k)):
        _check_on(name, t, q.device)
    _check_given("lse", lse, (Hq, total_q), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if validate:
        _check_max_seqlen(cu_seqlens_q, max_seqlen_q, "max_seqlen_q")
        _check_max_seqlen(cu_seqlens_k, max_seqlen_k, "max_seqlen_k")
    need = bwd_workspace_bytes(B, int(max_seqlen_q), Hq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_on("workspace", workspace, q.device)
    _check_given("dq", dq, q.shape, q.dtype, q.device)
    _check_given("dk", dk, k.shape, k.dtype, q.device)
    _check_given("dv", dv, v.shape, v.dtype, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    with torch.cuda.device(q.device):
        st = load().fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                  dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, int(max_seqlen_q),
                                  int(max_seqlen_k), total_q, total_k, Hq, Hkv, d, int(bool(causal)),
                                  float(scale), _dtype_code(q), workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), _stream(q))
    if st != 0:
        raise FaError(st, "fa_bwd_varlen")
    return dq, dk, dv


def _autograd_function():
    torch = _torch()

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, causal, scale, window):
            o, lse = attention(q, k, v, causal=causal, scale=scale, window=window)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.causal, ctx.scale, ctx.window = causal, scale, window
            return o

        @staticmethod
        def backward(ctx, dout):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv = attention_backward(q, k, v, o, lse, dout.contiguous(), causal=ctx.causal,
                                            scale=ctx.scale, window=ctx.window)
            return dq, dk, dv, None, None, None

    return _Attention


_ATTN_FN = None


def attention_func(q, k, v, causal: bool = False, scale: float | None = None, window=(-1, -1)):
    """attention(...)[0] as a differentiable torch op (forward and backward in libfa)."""
    global _ATTN_FN
    if _ATTN_FN is None:
        _ATTN_FN = _autograd_function()
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _ATTN_FN.apply(q, k, v, bool(causal), float(scale), tuple(int(x) for x in window))
