"""Exact FlashAttention-style attention forward for AMD MI355X (gfx950).

Thin binding over libattn.so (C ABI in include/attn.h): argument marshalling
only.  torch supplies device memory and the current stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: a
missing library or a non-GPU tensor raises.

    o, lse = prefill(q, k, v, causal=True)             # q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D]
    o, lse = decode_paged(q, k_cache, v_cache, block_table, ctx_lens, num_splits=0)
"""
from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import AttnError, MAX_SPLITS  # noqa: F401

__all__ = ["prefill", "prefill_paged", "decode_paged", "decode_paged_multi", "decode_paged_fp8",
           "decode_paged_noalloc", "decode_num_splits", "decode_workspace_bytes",
           "decode_workspace", "AttnError", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _stream_handle(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.ATTN_BF16
    if t.dtype == torch.float32:
        return _lib.ATTN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _need_gpu(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("attention_flash_fwd_amd runs on the GPU only; got a CPU tensor")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _same_device(ref, *ts):
    for t in ts:
        if t is not None and t.device != ref.device:
            raise ValueError(f"all tensors must be on {ref.device}; got one on {t.device}")


def _check_out(t, shape, dtype, name):
    """A caller-supplied output must have exactly the shape and dtype the
    kernels write: the C ABI takes raw pointers and cannot see a short or
    mistyped buffer, so this is the last place that can refuse one."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}; expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(ws):
    # The library checks the workspace's byte count itself; it must be one
    # flat byte buffer so that numel() is that count.
    if ws is not None and (ws.dim() != 1 or ws.element_size() != 1 or not ws.is_contiguous()):
        raise ValueError("workspace must be a contiguous 1-D byte tensor (see decode_workspace)")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() > 0 else 0)


def prefill(q, k, v, causal: bool = True, scale: float | None = None, out=None, lse_out=None,
            return_lse: bool = True):
    """Exact attention forward.  q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], bf16 or fp32.

    Returns (o [B,Sq,Hq,D] in q's dtype, lse [B,Hq,Sq] fp32 or None)."""
    import torch
    lib = _lib.load()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,Sq,Hq,D] and k, v [B,Sk,Hkv,D]")
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v disagree in batch, head_dim or dtype")
    _check_out(out, q.shape, q.dtype, "out")
    _check_out(lse_out, (B, Hq, Sq), torch.float32, "lse_out")
    _need_gpu(q, k, v, out, lse_out)
    _same_device(q, k, v, out, lse_out)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    st = lib.attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                          B, Sq, Sk, Hq, Hkv, D, int(bool(causal)), float(scale),
                          _dtype_code(q), _stream_handle(q))
    if st != _lib.ATTN_OK:
        raise AttnError(st, "attn_prefill")
    return o, lse


def decode_num_splits(batch, n_kv_heads, max_blocks_per_seq, block_size=16, num_splits=0) -> int:
    return int(_lib.load().attn_decode_num_splits(batch, n_kv_heads, max_blocks_per_seq,
                                                  block_size, num_splits))


def decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_blocks_per_seq,
                           block_size=16, num_splits=0) -> int:
    return int(_lib.load().attn_decode_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim,
                                                       max_blocks_per_seq, block_size, num_splits))


def decode_workspace(q, k_cache, block_table, num_splits=0):
    """Allocate a workspace tensor sized for these decode arguments (q is
    [B,Hq,D] for decode_paged or [B,T,Hq,D] for decode_paged_multi)."""
    import torch
    if q.dim() == 3:
        B, Hq, D = q.shape
        T = 1
    else:
        B, T, Hq, D = q.shape
    nbytes = int(_lib.load().attn_decode_multi_workspace_bytes(B, T, Hq, k_cache.shape[2], D,
                                                               block_table.shape[1], k_cache.shape[1],
                                                               num_splits))
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)


def prefill_paged(q, k_cache, v_cache, block_table, ctx_lens, causal: bool = True,
                  scale: float | None = None, out=None, lse_out=None, return_lse: bool = True):
    """A chunk of Sq new query tokens per sequence over a paged bf16 KV cache
    that already holds the chunk's own keys (chunked prefill).

    q [B,Sq,Hq,D]; k_cache/v_cache [num_blocks,16,Hkv,D]; block_table
    [B,max_blocks] int32; ctx_lens [B] int32 (keys per sequence, chunk
    included).  Returns (o [B,Sq,Hq,D] bf16, lse [B,Hq,Sq] fp32 or None)."""
    import torch
    lib = _lib.load()
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("prefill_paged takes bf16 q and caches")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("block_table and ctx_lens must be int32")
    if q.dim() != 4 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [B,Sq,Hq,D], caches [num_blocks,16,Hkv,D], block_table [B,max_blocks]")
    B, Sq, Hq, D = q.shape
    nblocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("inconsistent prefill_paged shapes")
    _check_out(out, q.shape, torch.bfloat16, "out")
    _check_out(lse_out, (B, Hq, Sq), torch.float32, "lse_out")
    _need_gpu(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out)
    _same_device(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    st = lib.attn_prefill_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                _ptr(ctx_lens), _ptr(o), _ptr(lse),
                                B, Sq, Hq, Hkv, D, nblocks, bs, block_table.shape[1],
                                1 if causal else 0, float(scale), _stream_handle(q))
    if st != _lib.ATTN_OK:
        raise AttnError(st, "attn_prefill_paged")
    return o, lse


def decode_paged_multi(q, k_cache, v_cache, block_table, ctx_lens, num_splits: int = 0,
                       scale: float | None = None, out=None, lse_out=None, workspace=None,
                       return_lse: bool = True):
    """T new query tokens per sequence (causal among themselves) over a paged
    bf16 KV cache that already holds their keys, as in speculative-decoding
    verification.  q [B,T,Hq,D]; other arguments as for decode_paged.
    Returns (o [B,T,Hq,D] bf16, lse [B,Hq,T] fp32 or None)."""
    import torch
    lib = _lib.load()
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("decode_paged_multi takes bf16 q and caches")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("block_table and ctx_lens must be int32")
    if q.dim() != 4 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [B,T,Hq,D], caches [num_blocks,16,Hkv,D], block_table [B,max_blocks]")
    B, T, Hq, D = q.shape
    nblocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("inconsistent decode shapes")
    _check_out(out, q.shape, torch.bfloat16, "out")
    _check_out(lse_out, (B, Hq, T), torch.float32, "lse_out")
    _check_workspace(workspace)
    _need_gpu(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out, workspace)
    _same_device(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = decode_workspace(q, k_cache, block_table, num_splits)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged_multi(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                     _ptr(ctx_lens), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D, nblocks, bs,
                                     block_table.shape[1], int(num_splits), float(scale),
                                     _ptr(workspace), workspace.numel(), _stream_handle(q))
    if st != _lib.ATTN_OK:
        raise AttnError(st, "attn_decode_paged_multi")
    return o, lse


def decode_paged_fp8(q, k_cache, v_cache, block_table, ctx_lens, k_scale: float, v_scale: float,
                     num_splits: int = 0, scale: float | None = None, out=None, lse_out=None,
                     workspace=None, return_lse: bool = True):
    """Decode over an FP8 (OCP e4m3) paged KV cache with per-tensor scales:
    K = e4m3(k_cache) * k_scale, V = e4m3(v_cache) * v_scale.  q [B,Hq,D] (one
    token) or [B,T,Hq,D]; caches uint8 [num_blocks,16,Hkv,D] holding e4m3
    codes.  Returns (o, lse) shaped like decode_paged / decode_paged_multi."""
    import torch
    lib = _lib.load()
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise TypeError("decode_paged_fp8 takes bf16 q and uint8 (e4m3) caches")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("block_table and ctx_lens must be int32")
    if q.dim() not in (3, 4) or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [B,Hq,D] or [B,T,Hq,D], caches [num_blocks,16,Hkv,D], "
                         "block_table [B,max_blocks]")
    single = q.dim() == 3
    q4 = q[:, None] if single else q
    B, T, Hq, D = q4.shape
    nblocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("inconsistent decode shapes")
    _check_out(out, q.shape, torch.bfloat16, "out")
    _check_out(lse_out, (B, Hq) if single else (B, Hq, T), torch.float32, "lse_out")
    _check_workspace(workspace)
    _need_gpu(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out, workspace)
    _same_device(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if workspace is None:
        workspace = decode_workspace(q4, k_cache, block_table, num_splits)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq) if single else (B, Hq, T), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged_fp8(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                   _ptr(ctx_lens), _ptr(o), _ptr(lse), B, T, Hq, Hkv, D, nblocks, bs,
                                   block_table.shape[1], int(num_splits), float(scale), float(k_scale),
                                   float(v_scale), _ptr(workspace), workspace.numel(), _stream_handle(q))
    if st != _lib.ATTN_OK:
        raise AttnError(st, "attn_decode_paged_fp8")
    return o, lse


def decode_paged(q, k_cache, v_cache, block_table, ctx_lens, num_splits: int = 0,
                 scale: float | None = None, out=None, lse_out=None, workspace=None,
                 return_lse: bool = True):
    """One query token per sequence over a paged bf16 KV cache.

    q [B,Hq,D]; k_cache/v_cache [num_blocks,16,Hkv,D]; block_table [B,max_blocks]
    int32; ctx_lens [B] int32.  Returns (o [B,Hq,D] bf16, lse [B,Hq] fp32 or None)."""
    import torch
    lib = _lib.load()
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("decode_paged takes bf16 q and caches")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("block_table and ctx_lens must be int32")
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [B,Hq,D], caches [num_blocks,16,Hkv,D], block_table [B,max_blocks]")
    B, Hq, D = q.shape
    nblocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("inconsistent decode shapes")
    _check_out(out, q.shape, torch.bfloat16, "out")
    _check_out(lse_out, (B, Hq), torch.float32, "lse_out")
    _check_workspace(workspace)
    _need_gpu(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out, workspace)
    _same_device(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out, workspace)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    max_blocks = block_table.shape[1]
    if workspace is None:
        workspace = decode_workspace(q, k_cache, block_table, num_splits)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                               _ptr(ctx_lens), _ptr(o), _ptr(lse),
                               B, Hq, Hkv, D, nblocks, bs, max_blocks, int(num_splits),
                               float(scale), _ptr(workspace), workspace.numel(),
                               _stream_handle(q))
    if st != _lib.ATTN_OK:
        raise AttnError(st, "attn_decode_paged")
    return o, lse


def decode_paged_noalloc(q, k_cache, v_cache, block_table, ctx_lens, num_splits: int = 0,
                         scale: float | None = None, out=None, lse_out=None, return_lse: bool = True):
    """decode_paged without a workspace: the library uses its own device
    array (attn_decode_paged_noalloc; the call itself allocates nothing, so
    pass `out` and `lse_out` to allocate nothing here either).  Calls that
    overlap in time on one GPU share that array and race.  Raises AttnError
    (ATTN_ERR_WORKSPACE) when the shape needs more than the array holds."""
    import torch
    lib = _lib.load()
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16 or v_cache.dtype != torch.bfloat16:
        raise TypeError("decode_paged_noalloc takes bf16 q and caches")
    if block_table.dtype != torch.int32 or ctx_lens.dtype != torch.int32:
        raise TypeError("block_table and ctx_lens must be int32")
    if q.dim() != 3 or k_cache.dim() != 4 or block_table.dim() != 2:
        raise ValueError("expected q [B,Hq,D], caches [num_blocks,16,Hkv,D], block_table [B,max_blocks]")
    B, Hq, D = q.shape
    nblocks, bs, Hkv, Dk = k_cache.shape
    if Dk != D or v_cache.shape != k_cache.shape or block_table.shape[0] != B or ctx_lens.shape != (B,):
        raise ValueError("inconsistent decode shapes")
    _check_out(out, q.shape, torch.bfloat16, "out")
    _check_out(lse_out, (B, Hq), torch.float32, "lse_out")
    _need_gpu(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out)
    _same_device(q, k_cache, v_cache, block_table, ctx_lens, out, lse_out)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = out if out is not None else torch.empty_like(q)
    lse = lse_out
    if lse is None and return_lse:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    st = lib.attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                       _ptr(ctx_lens), _ptr(o), _ptr(lse), B, Hq, Hkv, D, nblocks, bs,
                                       block_table.shape[1], int(num_splits), float(scale),
                                       _stream_handle(q))
    if st != _lib.ATTN_OK:
        raise AttnError(st, "attn_decode_paged_noalloc")
    return o, lse
