"""Exact fused attention for AMD Instinct MI355X (gfx950).

A thin binding over the C ABI of ``libfa.so`` (declared in include/fa.h):
argument marshalling only.  Every step of forward, backward and paged decode
runs in the library's HIP kernels; PyTorch supplies device memory and the
current stream.  There is no fallback: if the library is missing or a call
fails, a RuntimeError is raised.

    o, lse = forward(q, k, v, causal=True)            # q,k,v [B,H,N,d] bf16/fp32
    dq, dk, dv = backward(q, k, v, o, do, lse, causal=True)
    o, lse = decode_paged(q, kv_pool, block_table, seq_lens)
    o, lse = prefill_paged(q, kv_pool, block_table, seq_lens, cu_seqlens_q, max_q)

The softmax scale defaults to 1/sqrt(d), the default of the explainer pages
(lqnn.cn "为什么Flash突然成了AI圈的高频词" §3.3).
"""
from __future__ import annotations

import math

from ._lib import (  # noqa: F401
    FA_BF16,
    FA_F32,
    FaError,
    lib,
    library_path,
    status_name,
)

__all__ = [
    "forward",
    "backward",
    "forward_varlen",
    "backward_varlen",
    "decode_paged",
    "prefill_paged",
    "forward_rope",
    "backward_workspace_bytes",
    "decode_workspace_bytes",
    "FaError",
    "lib",
    "library_path",
]


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_dev(*ts):
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("all tensors must live on the GPU")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _expect(t, shape, dtype, name):
    """Check a caller-supplied tensor's shape and dtype before any launch: an
    undersized or mistyped buffer would otherwise be read or written past its
    end by the kernels."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _call(rc):
    if rc != 0:
        raise FaError(rc)


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
            return_lse: bool = True):
    """Fused forward; q [B, H, N, d], k/v [B, Hkv, N, d] (Hkv divides H: grouped
    key/value heads when Hkv < H).  Returns (o [B, H, N, d], lse fp32 [B, H, N] or None)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or Hkv == 0 or H % Hkv:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not return_lse:
        lse = None
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (B, H, N), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, o, lse)
    with torch.cuda.device(q.device):
        if Hkv == H:
            rc = lib().fa_forward(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  int(bool(causal)), float(scale), _stream(q))
        else:
            rc = lib().fa_forward_gqa(_dtype_code(q), B, H, Hkv, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                      int(bool(causal)), float(scale), _stream(q))
        _call(rc)
    return o, lse


def forward_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, scale: float | None = None,
                   out=None, lse=None, return_lse: bool = True):
    """Packed variable-length forward: q [total, H, d], k/v [total, Hkv, d],
    cu_seqlens int32 [B+1] on the GPU (sequence b = rows cu[b]..cu[b+1]-1).
    max_seqlen must be >= every length (cu_seqlens is not read on the host):
    a longer sequence is not computed past max_seqlen and its written rows
    are NaN in o and lse.
    Returns (o [total, H, d], lse fp32 [H, total] or None)."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
        raise ValueError("q must be [total, H, d] and k, v [total, Hkv, d]")
    if cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32 [B+1]")
    total, H, d = q.shape
    Hkv = k.shape[1]
    B = cu_seqlens.numel() - 1
    if Hkv == 0 or H % Hkv:
        raise ValueError("k, v must be [total, Hkv, d] with Hkv dividing H")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not return_lse:
        lse = None
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (H, total), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, cu_seqlens, o, lse)
    with torch.cuda.device(q.device):
        _call(lib().fa_forward_varlen(_dtype_code(q), B, H, Hkv, int(max_seqlen), total, d, _ptr(cu_seqlens), _ptr(q),
                                      _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(bool(causal)), float(scale),
                                      _stream(q)))
    return o, lse


def backward_workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().fa_backward_workspace_bytes(B, H, N, d))


def backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, workspace=None,
             dq=None, dk=None, dv=None):
    """Recomputing backward; returns (dq, dk, dv) bf16 with dk, dv shaped like k, v
    (grouped key/value heads sum their query heads' gradients)."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d or Hkv == 0 or H % Hkv:
        raise ValueError("k, v must be [B, Hkv, N, d] with Hkv dividing H")
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("o, dout must be shaped like q and v like k")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share a dtype")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [B, H, N]")
    _expect(dq, q.shape, q.dtype, "dq")
    _expect(dk, k.shape, q.dtype, "dk")
    _expect(dv, v.shape, q.dtype, "dv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = backward_workspace_bytes(B, H, N, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_dev(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    wsb = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        if Hkv == H:
            rc = lib().fa_backward(_dtype_code(q), B, H, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout),
                                   _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), wsb, int(bool(causal)),
                                   float(scale), _stream(q))
        else:
            rc = lib().fa_backward_gqa(_dtype_code(q), B, H, Hkv, N, d, _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                       _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), wsb,
                                       int(bool(causal)), float(scale), _stream(q))
        _call(rc)
    return dq, dk, dv


def backward_varlen(q, k, v, o, dout, lse, cu_seqlens, max_seqlen: int, causal: bool = False,
                    scale: float | None = None, workspace=None, dq=None, dk=None, dv=None):
    """Backward of forward_varlen (same packed layouts; lse fp32 [H, total]);
    max_seqlen as there (a longer sequence gets NaN gradients)."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q must be [total, H, d] and k, v [total, Hkv, d]")
    total, H, d = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != total or k.shape[2] != d or Hkv == 0 or H % Hkv:
        raise ValueError("k, v must be [total, Hkv, d] with Hkv dividing H")
    if o.shape != q.shape or dout.shape != q.shape or v.shape != k.shape:
        raise ValueError("o, dout must be shaped like q and v like k")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share a dtype")
    if cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32 [B+1]")
    B = cu_seqlens.numel() - 1
    if lse.shape != (H, total) or lse.dtype != torch.float32:
        raise ValueError("lse must be fp32 [H, total]")
    _expect(dq, q.shape, q.dtype, "dq")
    _expect(dk, k.shape, q.dtype, "dk")
    _expect(dv, v.shape, q.dtype, "dv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = int(lib().fa_backward_varlen_workspace_bytes(H, total, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_dev(q, k, v, o, dout, lse, cu_seqlens, dq, dk, dv, workspace)
    with torch.cuda.device(q.device):
        _call(lib().fa_backward_varlen(_dtype_code(q), B, H, Hkv, int(max_seqlen), total, d, _ptr(cu_seqlens),
                                       _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       int(bool(causal)), float(scale), _stream(q)))
    return dq, dk, dv


def decode_workspace_bytes(num_seqs: int, H: int, d: int, max_blocks: int) -> int:
    return int(lib().fa_decode_workspace_bytes(num_seqs, H, d, max_blocks))


def decode_paged(q, kv_pool, block_table, seq_lens, scale: float | None = None, workspace=None, out=None,
                 lse=None, return_lse: bool = True):
    """Paged decode; q [S, H, d] bf16, kv_pool [P, 2, page, Hkv, d] bf16 (Hkv
    divides H: grouped key/value heads when Hkv < H), block_table
    [S, max_blocks] int32, seq_lens [S] int32 (all on the GPU).
    Returns (o [S, H, d] bf16, lse [S, H] fp32 or None)."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [S, H, d]")
    S, H, d = q.shape
    if (kv_pool.dim() != 5 or kv_pool.shape[1] != 2 or kv_pool.shape[4] != d or kv_pool.shape[3] == 0
            or H % kv_pool.shape[3]):
        raise ValueError("kv_pool must be [pages, 2, page_size, Hkv, d] with Hkv dividing H")
    if block_table.dim() != 2 or block_table.shape[0] != S or block_table.dtype != torch.int32:
        raise ValueError("block_table must be int32 [S, max_blocks]")
    if seq_lens.shape != (S,) or seq_lens.dtype != torch.int32:
        raise ValueError("seq_lens must be int32 [S]")
    if q.dtype != torch.bfloat16 or kv_pool.dtype != torch.bfloat16:
        raise TypeError("paged decode takes bf16 q and kv_pool")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    P, _, page, Hkv, _ = kv_pool.shape
    mb = block_table.shape[1]
    if not return_lse:
        lse = None
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (S, H), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((S, H), dtype=torch.float32, device=q.device)
    need = decode_workspace_bytes(S, H, d, mb)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_dev(q, kv_pool, block_table, seq_lens, o, lse, workspace)
    wsb = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        if Hkv == H:
            rc = lib().fa_decode_paged(S, H, d, page, P, mb, _ptr(q), _ptr(kv_pool), _ptr(block_table),
                                       _ptr(seq_lens), _ptr(o), _ptr(lse), float(scale), _ptr(workspace), wsb,
                                       _stream(q))
        else:
            rc = lib().fa_decode_paged_gqa(S, H, Hkv, d, page, P, mb, _ptr(q), _ptr(kv_pool), _ptr(block_table),
                                           _ptr(seq_lens), _ptr(o), _ptr(lse), float(scale), _ptr(workspace), wsb,
                                           _stream(q))
        _call(rc)
    return o, lse


def _rope_args(rope_cos, rope_sin, d):
    torch = _torch()
    if rope_cos is None and rope_sin is None:
        return None, None, 0
    if rope_cos is None or rope_sin is None:
        raise ValueError("pass both rotary tables or neither")
    for t in (rope_cos, rope_sin):
        if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != d // 2:
            raise ValueError("rotary tables must be fp32 [rows, d/2]")
    if rope_cos.shape != rope_sin.shape:
        raise ValueError("rotary tables must have the same shape")
    return rope_cos, rope_sin, rope_cos.shape[0]


def forward_rope(q, k, v, rope_cos, rope_sin, causal: bool = False, scale: float | None = None,
                 interleaved: bool = False, cu_seqlens=None, max_seqlen: int | None = None, out=None, lse=None,
                 return_lse: bool = True):
    """Forward with the rotary embedding of Q and K fused into the kernel.
    Dense: q [B, H, N, d], k/v [B, Hkv, N, d]; packed (cu_seqlens given):
    q [total, H, d], k/v [total, Hkv, d].  rope_cos / rope_sin fp32
    [rows, d/2] with rows >= N (max_seqlen): position p rotates feature pair
    i (i, i + d/2), or (2i, 2i+1) when interleaved, by cos[p][i], sin[p][i].
    Returns (o, lse) laid out as forward / forward_varlen."""
    torch = _torch()
    packed = cu_seqlens is not None
    if packed:
        if q.dim() != 3 or k.dim() != 3 or k.shape[0] != q.shape[0] or k.shape[2] != q.shape[2]:
            raise ValueError("packed q must be [total, H, d] and k, v [total, Hkv, d]")
        if cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32 or max_seqlen is None:
            raise ValueError("packed form needs cu_seqlens int32 [B+1] and max_seqlen")
        total, H, d = q.shape
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        N = int(max_seqlen)
        lse_shape = (H, total)
    else:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("q must be [B, H, N, d] and k, v [B, Hkv, N, d]")
        B, H, N, d = q.shape
        Hkv = k.shape[1]
        if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
            raise ValueError("k, v must be [B, Hkv, N, d]")
        total = 0
        lse_shape = (B, H, N)
    if Hkv == 0 or H % Hkv:
        raise ValueError("the key/value heads must divide the query heads")
    if v.shape != k.shape:
        raise ValueError("k and v must have the same shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    cos_t, sin_t, rows = _rope_args(rope_cos, rope_sin, d)
    if cos_t is None:
        raise ValueError("forward_rope needs the rotary tables")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not return_lse:
        lse = None
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, lse_shape, torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty(lse_shape, dtype=torch.float32, device=q.device)
    _check_dev(q, k, v, cos_t, sin_t, o, lse, *( [cu_seqlens] if packed else [] ))
    with torch.cuda.device(q.device):
        _call(lib().fa_forward_rope(_dtype_code(q), B, H, Hkv, N, total, d, _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(o), _ptr(lse), int(bool(causal)), float(scale), _ptr(cos_t),
                                    _ptr(sin_t), rows, int(bool(interleaved)), _stream(q)))
    return o, lse


def prefill_paged(q, kv_pool, block_table, seq_lens_k, cu_seqlens_q, max_seqlen_q: int, causal: bool = True,
                  scale: float | None = None, out=None, lse=None, return_lse: bool = True, rope_cos=None,
                  rope_sin=None, rope_interleaved: bool = False):
    """Chunked prefill over a paged KV cache: q [total_q, H, d] bf16 (the new
    chunk of every sequence, packed by cu_seqlens_q int32 [B+1]); kv_pool
    [P, 2, page, Hkv, d] bf16 holding each sequence's seq_lens_k[b] keys
    (prefix, then the chunk) through block_table [B, max_blocks] int32.
    Causal: query i of a chunk of n sees keys 0 .. i + seq_lens_k[b] - n.
    With rotary tables the queries are rotated at those positions (the cached
    keys are taken as stored, already rotated).
    Returns (o [total_q, H, d] bf16, lse [H, total_q] fp32 or None)."""
    torch = _torch()
    if q.dim() != 3 or kv_pool.dim() != 5 or kv_pool.shape[1] != 2 or kv_pool.shape[4] != q.shape[2]:
        raise ValueError("q must be [total_q, H, d] and kv_pool [pages, 2, page_size, Hkv, d]")
    total, H, d = q.shape
    P, _, page, Hkv, _ = kv_pool.shape
    B = cu_seqlens_q.numel() - 1
    if Hkv == 0 or H % Hkv:
        raise ValueError("the pool's key/value heads must divide the query heads")
    if cu_seqlens_q.dtype != torch.int32 or seq_lens_k.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("cu_seqlens_q, seq_lens_k and block_table must be int32")
    if seq_lens_k.shape != (B,) or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("seq_lens_k must be [B] and block_table [B, max_blocks]")
    if q.dtype != torch.bfloat16 or kv_pool.dtype != torch.bfloat16:
        raise TypeError("paged prefill takes bf16 q and kv_pool")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if not return_lse:
        lse = None
    _expect(out, q.shape, q.dtype, "out")
    _expect(lse, (H, total), torch.float32, "lse")
    o = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    cos_t, sin_t, rows = _rope_args(rope_cos, rope_sin, d)
    _check_dev(q, kv_pool, block_table, seq_lens_k, cu_seqlens_q, o, lse, cos_t, sin_t)
    with torch.cuda.device(q.device):
        _call(lib().fa_prefill_paged(B, H, Hkv, d, int(max_seqlen_q), total, _ptr(cu_seqlens_q), _ptr(q),
                                     _ptr(kv_pool), page, P, _ptr(block_table), block_table.shape[1],
                                     _ptr(seq_lens_k), _ptr(o), _ptr(lse), int(bool(causal)), float(scale),
                                     _ptr(cos_t), _ptr(sin_t), rows, int(bool(rope_interleaved)), _stream(q)))
    return o, lse
