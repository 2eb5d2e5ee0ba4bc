"""Torch-facing wrappers of the C ABI: dash.summarize / route / route_topk /
attn_prefill / attn_sparse / attn_decode / attn_decode_sparse.

Torch supplies device memory (inputs, outputs, the workspace) and the current
stream; every computation runs in libdash.so.  Shapes follow include/dash.h:
token-major q [T, Hq, D], k/v [T, Hkv, D]; decode caches [batch, cap, Hkv, D].
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return L.DASH_BF16
    if t.dtype == torch.float32:
        return L.DASH_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("dash ops take GPU tensors")
            if not t.is_contiguous():
                raise ValueError("dash ops take contiguous tensors")


def _seq_shape(q_or_k, num_heads_q, num_heads_kv, chunk_size, cu_seqlens, max_seqlen):
    T, _, D = q_or_k.shape
    if cu_seqlens is None:
        num_seqs = 1 if max_seqlen is None else T // max_seqlen
        max_seqlen = T if max_seqlen is None else max_seqlen
        cu_ptr = None
    else:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        num_seqs = cu_seqlens.numel() - 1
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        cu_ptr = cu_seqlens.data_ptr()
    return L.make_shape(num_seqs, max_seqlen, T, cu_ptr, num_heads_q, num_heads_kv, D,
                        chunk_size, _dtype_code(q_or_k))


def _workspace(op, shape, device):
    n = L.workspace_size(op, shape)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    return ws, n


def layout(shape, enable_gqa=True):
    return L.layout(shape, enable_gqa)


def summarize(k, qbar, chunk_size, cu_seqlens=None, max_seqlen=None, out=None,
              workspace=None):
    """Phase-0 chunk summaries; returns k_bar [floor(T/B), Hkv, D] (k's dtype)."""
    _need_cuda(k, qbar, cu_seqlens)
    T, Hkv, D = k.shape
    shape = _seq_shape(k, Hkv, Hkv, chunk_size, cu_seqlens, max_seqlen)
    if out is None:
        lay = L.layout(shape)
        out = torch.empty((lay.summary_rows, Hkv, D), dtype=k.dtype, device=k.device)
    if workspace is None:
        ws, n = _workspace(L.DASH_OP_SUMMARIZE, shape, k.device)
    else:
        # a caller's workspace is used only when it is large enough
        n = L.workspace_size(L.DASH_OP_SUMMARIZE, shape)
        ws = workspace if workspace.numel() >= n else _workspace(L.DASH_OP_SUMMARIZE, shape, k.device)[0]
    L.check("dash_summarize", L.lib().dash_summarize(
        ctypes.byref(shape), _ptr(k), _ptr(qbar.float().contiguous() if qbar.dtype != torch.float32 else qbar),
        _ptr(out), _ptr(ws), n, _stream(k.device)))
    return out


def summarize_diagonal(k, qbar, chunk_size, cu_seqlens=None, max_seqlen=None, out=None):
    """Estimated summary of every position's own partial chunk (for
    estimate_diagonal routing); returns k_diag [T, Hkv, D] (k's dtype)."""
    _need_cuda(k, qbar, cu_seqlens)
    T, Hkv, D = k.shape
    shape = _seq_shape(k, Hkv, Hkv, chunk_size, cu_seqlens, max_seqlen)
    if out is None:
        out = torch.empty_like(k)
    qb = qbar if qbar.dtype == torch.float32 else qbar.float().contiguous()
    L.check("dash_summarize_diagonal", L.lib().dash_summarize_diagonal(
        ctypes.byref(shape), _ptr(k), _ptr(qb), _ptr(out), _stream(k.device)))
    return out


def route(q, kbar, num_kv_heads, chunk_size, *, alpha=1.5, gamma=1.0, sigma=1.0,
          softmax_scale=0.0, enable_gqa=True, alpha_per_seq=None, cu_seqlens=None,
          max_seqlen=None, log_prior=False, tau=False, mask_out=None, log_prior_out=None,
          workspace=None, kdiag=None):
    """Phase-1 routing.  Returns (active_blocks [Hkv,T,W] int64 view of the
    uint64 words, log_prior [Hkv,T,C_slots] or None, tau [Hq,T] or None).
    kdiag [T, Hkv, D] (summarize_diagonal) adds each row's own-chunk estimate
    to its entmax."""
    _need_cuda(q, kbar, alpha_per_seq, cu_seqlens, mask_out, log_prior_out, kdiag)
    T, Hq, D = q.shape
    shape = _seq_shape(q, Hq, num_kv_heads, chunk_size, cu_seqlens, max_seqlen)
    dev = q.device
    if mask_out is None or (log_prior and log_prior_out is None):
        lay = L.layout(shape, enable_gqa)
    mask = mask_out if mask_out is not None else torch.empty(
        (num_kv_heads, T, lay.mask_words), dtype=torch.int64, device=dev)
    if log_prior_out is not None:
        lp = log_prior_out
    else:
        lp = (torch.full((num_kv_heads, T, lay.chunk_slots), float("nan"), device=dev)
              if log_prior else None)
    ta = torch.empty((Hq, T), dtype=torch.float32, device=dev) if tau else None
    if workspace is None:
        ws, n = _workspace(L.DASH_OP_ROUTE, shape, dev)
    else:
        # a caller's workspace is used only when it is large enough
        n = L.workspace_size(L.DASH_OP_ROUTE, shape)
        ws = workspace if workspace.numel() >= n else _workspace(L.DASH_OP_ROUTE, shape, dev)[0]
    L.check("dash_route", L.lib().dash_route(
        ctypes.byref(shape), _ptr(q), _ptr(kbar), _ptr(kdiag), float(alpha), _ptr(alpha_per_seq),
        float(gamma), float(sigma), float(softmax_scale), int(enable_gqa), _ptr(mask),
        _ptr(lp), _ptr(ta), _ptr(ws), n, _stream(dev)))
    return mask, lp, ta


def route_topk(q, kbar, num_kv_heads, chunk_size, topk, *, gamma=1.0, softmax_scale=0.0,
               enable_gqa=True, cu_seqlens=None, max_seqlen=None, decode_seqlens=None,
               cache_len=None, log_prior=True, mask_out=None, log_prior_out=None,
               workspace=None):
    """Top-k block routing (the comparison mode).  Prefill rows as route();
    with decode_seqlens (int32 [batch]) one decode row per batch entry, q
    [batch, Hq, D], kbar the summary cache [batch, cache_len/B, Hkv, D].
    Returns (active_blocks int64 words, log_prior or None)."""
    _need_cuda(q, kbar, cu_seqlens, decode_seqlens, mask_out, log_prior_out)
    rows, Hq, D = q.shape
    dev = q.device
    if decode_seqlens is None:
        shape = _seq_shape(q, Hq, num_kv_heads, chunk_size, cu_seqlens, max_seqlen)
        lay = L.layout(shape, enable_gqa)
        op_ws = L.DASH_OP_ROUTE
    else:
        if cache_len is None:
            raise ValueError("cache_len is required with decode_seqlens")
        shape = L.make_shape(rows, cache_len, rows, None, Hq, num_kv_heads, D, chunk_size,
                             _dtype_code(q))
        lay = L.layout(L.make_shape(rows, cache_len, rows * cache_len, None, Hq, num_kv_heads,
                                    D, chunk_size, _dtype_code(q)), enable_gqa)
        op_ws = L.DASH_OP_ROUTE_DECODE
    mask = mask_out if mask_out is not None else torch.empty(
        (num_kv_heads, rows, lay.mask_words), dtype=torch.int64, device=dev)
    if log_prior_out is not None:
        lp = log_prior_out
    else:
        lp = (torch.full((num_kv_heads, rows, lay.chunk_slots), float("nan"), device=dev)
              if log_prior else None)
    if workspace is None:
        ws, n = _workspace(op_ws, shape, dev)
    else:
        # a caller's workspace is used only when it is large enough
        n = L.workspace_size(op_ws, shape)
        ws = workspace if workspace.numel() >= n else _workspace(op_ws, shape, dev)[0]
    L.check("dash_route_topk", L.lib().dash_route_topk(
        ctypes.byref(shape), _ptr(q), _ptr(kbar), int(topk), float(gamma),
        float(softmax_scale), int(enable_gqa), _ptr(decode_seqlens), _ptr(mask), _ptr(lp),
        _ptr(ws), n, _stream(dev)))
    return mask, lp


def route_topk_decode_workspace(q, num_kv_heads, chunk_size, cache_len):
    """Allocate the workspace route_topk needs for decode rows (q [batch, Hq, D])."""
    batch, Hq, D = q.shape
    shape = L.make_shape(batch, cache_len, batch, None, Hq, num_kv_heads, D, chunk_size,
                         _dtype_code(q))
    n = L.workspace_size(L.DASH_OP_ROUTE_DECODE, shape)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def attn_prefill(q, k, v, qbar, chunk_size, *, alpha=1.5, gamma=1.0, sigma=1.0,
                 softmax_scale=0.0, enable_gqa=True, alpha_per_seq=None, cu_seqlens=None,
                 max_seqlen=None, return_lse=False, return_active_blocks=False,
                 workspace=None, estimate_diagonal=False):
    """Phases 0-2, causal prefill.  Returns (out, lse or None, active_blocks or None).
    estimate_diagonal routes every row with its own-chunk estimate too."""
    _need_cuda(q, k, v, qbar, alpha_per_seq, cu_seqlens)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    shape = _seq_shape(q, Hq, Hkv, chunk_size, cu_seqlens, max_seqlen)
    lay = L.layout(shape, enable_gqa)
    dev = q.device
    out = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if return_lse else None
    ab = (torch.empty((Hkv, T, lay.mask_words), dtype=torch.int64, device=dev)
          if return_active_blocks else None)
    n = L.workspace_size(L.DASH_OP_PREFILL, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_prefill", L.lib().dash_attn_prefill(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(qbar), float(alpha),
        _ptr(alpha_per_seq), float(gamma), float(sigma), float(softmax_scale),
        int(enable_gqa), int(estimate_diagonal), _ptr(out), _ptr(lse), _ptr(ab),
        _ptr(workspace), n, _stream(dev)))
    return out, lse, ab


def attn_prefill_backward(q, k, v, qbar, out, dout, lse, chunk_size, *, alpha=1.5, gamma=1.0,
                          sigma=1.0, softmax_scale=0.0, enable_gqa=True, alpha_per_seq=None,
                          cu_seqlens=None, max_seqlen=None, estimate_diagonal=False,
                          workspace=None):
    """Backward of attn_prefill (fixed-length sequences of max_seqlen tokens,
    one of T if None, or packed by cu_seqlens): returns (dq, dk, dv, dqbar
    [Hkv, D] fp32)."""
    _need_cuda(q, k, v, qbar, out, dout, lse, alpha_per_seq, cu_seqlens)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    shape = _seq_shape(q, Hq, Hkv, chunk_size, cu_seqlens, max_seqlen)
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dqbar = torch.empty((Hkv, D), dtype=torch.float32, device=dev)
    qb = qbar if qbar.dtype == torch.float32 else qbar.float().contiguous()
    n = L.workspace_size(L.DASH_OP_PREFILL_BACKWARD, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_prefill_backward", L.lib().dash_attn_prefill_backward(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(qb), float(alpha),
        _ptr(alpha_per_seq), float(gamma), float(sigma), float(softmax_scale), int(enable_gqa),
        int(estimate_diagonal), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(dqbar),
        _ptr(workspace), n, _stream(dev)))
    return dq, dk, dv, dqbar


def attn_sparse_backward(q, k, v, out, dout, lse, active_blocks, log_prior, chunk_size, *,
                         softmax_scale=0.0, enable_gqa=True, cu_seqlens=None, max_seqlen=None,
                         workspace=None):
    """Backward of attn_sparse: returns (dq, dk, dv, dbias [Hkv, T, C_slots])."""
    _need_cuda(q, k, v, out, dout, lse, active_blocks, log_prior, cu_seqlens)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    shape = _seq_shape(q, Hq, Hkv, chunk_size, cu_seqlens, max_seqlen)
    lay = L.layout(shape, enable_gqa)
    dev = q.device
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dbias = torch.empty((Hkv, T, lay.chunk_slots), dtype=torch.float32, device=dev)
    n = L.workspace_size(L.DASH_OP_BACKWARD, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_sparse_backward", L.lib().dash_attn_sparse_backward(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
        _ptr(active_blocks), _ptr(log_prior), float(softmax_scale), int(enable_gqa), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(dbias), _ptr(workspace), n, _stream(dev)))
    return dq, dk, dv, dbias


def attn_sparse(q, k, v, active_blocks, log_prior, chunk_size, *, softmax_scale=0.0,
                enable_gqa=True, cu_seqlens=None, max_seqlen=None, return_lse=False,
                out=None, workspace=None):
    """Phase 2 alone for a given routing (active_blocks [Hkv,T,W] int64 words,
    log_prior [Hkv,T,C_slots] fp32).  Returns (out, lse or None)."""
    _need_cuda(q, k, v, active_blocks, log_prior, cu_seqlens)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    shape = _seq_shape(q, Hq, Hkv, chunk_size, cu_seqlens, max_seqlen)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, T), dtype=torch.float32, device=dev) if return_lse else None
    n = L.workspace_size(L.DASH_OP_SPARSE, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_sparse", L.lib().dash_attn_sparse(
        ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(active_blocks), _ptr(log_prior),
        float(softmax_scale), int(enable_gqa), _ptr(out), _ptr(lse), _ptr(workspace), n,
        _stream(dev)))
    return out, lse


def sparse_workspace(q, k, chunk_size, cu_seqlens=None, max_seqlen=None):
    """Allocate the workspace attn_sparse needs, for reuse across calls."""
    T, Hq, D = q.shape
    shape = _seq_shape(q, Hq, k.shape[1], chunk_size, cu_seqlens, max_seqlen)
    n = L.workspace_size(L.DASH_OP_SPARSE, shape)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def prefill_workspace(q, k, chunk_size, cu_seqlens=None, max_seqlen=None):
    """Allocate the workspace attn_prefill needs, for reuse across calls."""
    T, Hq, D = q.shape
    shape = _seq_shape(q, Hq, k.shape[1], chunk_size, cu_seqlens, max_seqlen)
    n = L.workspace_size(L.DASH_OP_PREFILL, shape)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def decode_shape(q, k_cache, chunk_size):
    batch, Hq, D = q.shape
    _, cap, Hkv, _ = k_cache.shape
    return L.make_shape(batch, cap, batch, None, Hq, Hkv, D, chunk_size, _dtype_code(q))


def attn_decode(q, k_cache, v_cache, seqlens, kbar_cache, chunk_size, *, alpha=1.5,
                gamma=1.0, sigma=1.0, softmax_scale=0.0, enable_gqa=True,
                return_lse=False, return_active_blocks=False, workspace=None, out=None,
                estimate_diagonal=False, qbar=None):
    """One decode step.  q [batch, Hq, D]; caches [batch, cap, Hkv, D];
    seqlens int32 [batch]; kbar_cache [batch, cap/B, Hkv, D].  With
    estimate_diagonal, qbar [Hkv, D] gives the new rows' own-chunk estimates."""
    if estimate_diagonal and qbar is None:
        raise ValueError("estimate_diagonal needs qbar")
    qb = None if qbar is None else (qbar if qbar.dtype == torch.float32
                                    else qbar.float().contiguous())
    _need_cuda(q, k_cache, v_cache, seqlens, kbar_cache, qb)
    batch, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    shape = decode_shape(q, k_cache, chunk_size)
    lay = L.layout(L.make_shape(batch, k_cache.shape[1], batch * k_cache.shape[1], None, Hq,
                                Hkv, D, chunk_size, _dtype_code(q)), enable_gqa)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, batch), dtype=torch.float32, device=dev) if return_lse else None
    ab = (torch.empty((Hkv, batch, lay.mask_words), dtype=torch.int64, device=dev)
          if return_active_blocks else None)
    n = L.workspace_size(L.DASH_OP_DECODE, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_decode", L.lib().dash_attn_decode(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens),
        _ptr(kbar_cache), _ptr(qb), float(alpha), float(gamma), float(sigma),
        float(softmax_scale), int(enable_gqa), int(estimate_diagonal), _ptr(out), _ptr(lse),
        _ptr(ab), _ptr(workspace), n, _stream(dev)))
    return out, lse, ab


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, seqlens, kbar_cache, qbar,
                       chunk_size, *, alpha=1.5, gamma=1.0, sigma=1.0, softmax_scale=0.0,
                       enable_gqa=True, return_lse=False, return_active_blocks=False,
                       workspace=None, out=None, estimate_diagonal=False):
    """dash_attn_decode_append: cache_append and attn_decode as one fused step.
    Writes the new tokens' K/V rows (k_new, v_new [batch, Hkv, D]) at position
    seqlens[b]-1 of the caches and the summary of each chunk they complete
    into kbar_cache, then decodes q over the updated caches."""
    qb = qbar if qbar.dtype == torch.float32 else qbar.float().contiguous()
    _need_cuda(q, k_new, v_new, k_cache, v_cache, seqlens, kbar_cache, qb)
    batch, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    shape = decode_shape(q, k_cache, chunk_size)
    lay = L.layout(L.make_shape(batch, k_cache.shape[1], batch * k_cache.shape[1], None, Hq,
                                Hkv, D, chunk_size, _dtype_code(q)), enable_gqa)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, batch), dtype=torch.float32, device=dev) if return_lse else None
    ab = (torch.empty((Hkv, batch, lay.mask_words), dtype=torch.int64, device=dev)
          if return_active_blocks else None)
    n = L.workspace_size(L.DASH_OP_DECODE, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_decode_append", L.lib().dash_attn_decode_append(
        ctypes.byref(shape), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
        _ptr(seqlens), _ptr(kbar_cache), _ptr(qb), float(alpha), float(gamma), float(sigma),
        float(softmax_scale), int(enable_gqa), int(estimate_diagonal), _ptr(out), _ptr(lse),
        _ptr(ab), _ptr(workspace), n, _stream(dev)))
    return out, lse, ab


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, kbar_cache, chunk_size, out, *,
                        alpha=1.5, gamma=1.0, sigma=1.0, softmax_scale=0.0, enable_gqa=True,
                        lse=None, active_blocks=None, estimate_diagonal=False, qbar=None):
    """dash_attn_decode_noalloc: one decode step whose intermediates live in the
    library's own per-device scratch (no workspace, nothing allocated here
    either: the caller passes out [batch, Hq, D] and, optionally, lse
    [Hq, batch] fp32 and active_blocks [Hkv, batch, W] int64)."""
    if estimate_diagonal and (qbar is None or qbar.dtype != torch.float32):
        raise ValueError("estimate_diagonal needs an fp32 qbar")
    _need_cuda(q, k_cache, v_cache, seqlens, kbar_cache, qbar, out, lse, active_blocks)
    shape = decode_shape(q, k_cache, chunk_size)
    L.check("dash_attn_decode_noalloc", L.lib().dash_attn_decode_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens),
        _ptr(kbar_cache), _ptr(qbar), float(alpha), float(gamma), float(sigma),
        float(softmax_scale), int(enable_gqa), int(estimate_diagonal), _ptr(out), _ptr(lse),
        _ptr(active_blocks), _stream(q.device)))
    return out


def decode_workspace(q, k_cache, chunk_size):
    n = L.workspace_size(L.DASH_OP_DECODE, decode_shape(q, k_cache, chunk_size))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def cache_append(k_new, v_new, seqlens, qbar, k_cache, v_cache, kbar_cache, chunk_size):
    """Decode-cache upkeep: write each batch entry's new key/value (k_new,
    v_new [batch, Hkv, D]) at position seqlens[b]-1 of the caches [batch, cap,
    Hkv, D] and, when that completes a chunk, its summary into kbar_cache
    [batch, cap/B, Hkv, D].  seqlens (int32 [batch]) are the lengths after the
    append.  Updates the caches in place."""
    _need_cuda(k_new, v_new, seqlens, qbar, k_cache, v_cache, kbar_cache)
    batch, cap, Hkv, D = k_cache.shape
    shape = L.make_shape(batch, cap, batch, None, Hkv, Hkv, D, chunk_size, _dtype_code(k_cache))
    qb = qbar if qbar.dtype == torch.float32 else qbar.float().contiguous()
    L.check("dash_cache_append", L.lib().dash_cache_append(
        ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(seqlens), _ptr(qb), _ptr(k_cache),
        _ptr(v_cache), _ptr(kbar_cache), _stream(k_cache.device)))


def decode_sparse_workspace(q, k_cache, chunk_size):
    n = L.workspace_size(L.DASH_OP_DECODE_SPARSE, decode_shape(q, k_cache, chunk_size))
    return torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)


def attn_decode_sparse(q, k_cache, v_cache, seqlens, active_blocks, log_prior, chunk_size, *,
                       softmax_scale=0.0, enable_gqa=True, return_lse=False, workspace=None,
                       out=None):
    """The attention step of a decode for a given routing (active_blocks
    [Hkv, batch, W] int64 words, log_prior [Hkv, batch, C_slots])."""
    _need_cuda(q, k_cache, v_cache, seqlens, active_blocks, log_prior)
    batch, Hq, D = q.shape
    shape = decode_shape(q, k_cache, chunk_size)
    dev = q.device
    if out is None:
        out = torch.empty_like(q)
    lse = torch.empty((Hq, batch), dtype=torch.float32, device=dev) if return_lse else None
    n = L.workspace_size(L.DASH_OP_DECODE_SPARSE, shape)
    if workspace is None or workspace.numel() < n:
        workspace = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    L.check("dash_attn_decode_sparse", L.lib().dash_attn_decode_sparse(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens),
        _ptr(active_blocks), _ptr(log_prior), float(softmax_scale), int(enable_gqa), _ptr(out),
        _ptr(lse), _ptr(workspace), n, _stream(dev)))
    return out, lse
