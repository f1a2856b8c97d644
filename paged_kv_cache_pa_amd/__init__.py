"""Paged-KV-cache attention for MI355X (gfx950): Python binding of libpa.so.

The functions mirror the C ABI in include/pa.h and take torch tensors that
already live on the GPU.  Torch supplies device memory and the current
stream; the library's HIP kernels do all the work, and nothing here has a
CPU fallback: a missing library raises ImportError on first use.
"""
from __future__ import annotations

import ctypes

from ._lib import (PA_BF16, PA_F16, PROFILE_KINDS, PAError, check, lib)  # noqa: F401

__all__ = ["pa_scatter_kv", "pa_scatter_kv_paged", "pa_scatter_kv_fp8", "pa_scatter_kv_paged_fp8",
           "pa_seqlens_from_past", "pa_attention", "pa_attention_rope", "pa_attention_noalloc",
           "pa_attention_fp8", "pa_attention_rope_fp8",
           "pa_rotary_scatter_kv", "pa_rotary_scatter_kv_fp8",
           "pa_attention_workspace_size", "pa_validate_metadata", "profile_enable",
           "profile_read", "PAError"]


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return PA_F16
    if t.dtype == torch.bfloat16:
        return PA_BF16
    raise ValueError(f"unsupported dtype {t.dtype} (float16 or bfloat16)")


def _stream_ptr(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _alloc_on(stream, ref, shape, dtype):
    """A new GPU tensor allocated on the stream the kernels will use, so that
    the caching allocator does not hand its bytes to other work on another
    stream while those kernels still run (the tensor may be dropped as soon
    as the call returns)."""
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(ref.device)
    with torch.cuda.stream(s):
        return torch.empty(shape, dtype=dtype, device=ref.device)


def _dev(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def pa_scatter_kv(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None):
    """Write new K/V rows [T, Hk, D] into the paged caches [NB, bs, Hk, D]
    at int32 ``slot_mapping`` [T] (negative = skip), in place."""
    import torch
    T, hk, d = k_new.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    if tuple(v_new.shape) != (T, hk, d) or tuple(k_cache.shape) != (nb, bs, hk, d) \
            or tuple(v_cache.shape) != (nb, bs, hk, d) or slot_mapping.shape != (T,):
        raise ValueError("inconsistent shapes")
    if not (k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("K/V and caches must share one dtype")
    check(lib().pa_scatter_kv(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), T, nb, hk, d, bs,
        _dtype_code(k_cache), _stream_ptr(k_cache, stream)))


def pa_scatter_kv_paged(k_new, v_new, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache,
                        stream=None):
    """pa_scatter_kv with the slots derived on the GPU: token t of sequence b
    goes to KV position past_b + (t - cu[b]) of b's block-table row."""
    import torch
    T, hk, d = k_new.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    if tuple(v_new.shape) != (T, hk, d) or tuple(k_cache.shape) != (nb, bs, hk, d) \
            or tuple(v_cache.shape) != (nb, bs, hk, d) or seqlens_kv.shape != (B,) \
            or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("inconsistent shapes")
    if not (k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("K/V and caches must share one dtype")
    check(lib().pa_scatter_kv_paged(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), B, T, block_table.shape[1], nb, hk, d,
        bs, _dtype_code(k_cache), _stream_ptr(k_cache, stream)))


def pa_seqlens_from_past(cu_seqlens_q, past_seqlens, out=None, stream=None):
    """Total KV lengths (int32 [B]) from past lengths: past[b] + q_len_b."""
    import torch
    B = cu_seqlens_q.shape[0] - 1
    if past_seqlens.shape != (B,):
        raise ValueError("inconsistent shapes")
    if out is None:
        out = _alloc_on(stream, past_seqlens, (B,), torch.int32)
    check(lib().pa_seqlens_from_past(
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(past_seqlens, "past_seqlens", torch.int32),
        _dev(out, "out", torch.int32), B, _stream_ptr(out, stream)))
    return out


def _rotary(query, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, num_heads,
            num_kv_heads, key, value, cos_cache, sin_cache, interleaved, q_out, stream, write_q,
            k_scale=None, v_scale=None):
    import torch
    kv8 = k_scale is not None or v_scale is not None
    if query is None and (write_q or key is None):
        raise ValueError("query may be None only with key/value given and write_q=False")
    ref = query if query is not None else key
    T = ref.shape[0]
    nb, bs, hk, d = k_cache.shape
    B = seqlens_kv.shape[0]
    MB = block_table.shape[1]
    if hk != num_kv_heads or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or cu_seqlens_q.shape != (B + 1,) or block_table.shape[0] != B:
        raise ValueError("inconsistent shapes")
    if key is None:
        if value is not None or query.numel() != T * (num_heads + 2 * num_kv_heads) * d:
            raise ValueError("packed QKV rows must hold Hq + 2 Hk heads")
    elif (query is not None and query.numel() != T * num_heads * d) or key.numel() != T * hk * d \
            or value is None or value.numel() != T * hk * d:
        raise ValueError("inconsistent Q/K/V shapes")
    caches = () if kv8 else (k_cache, v_cache)
    for t in (key, value, cos_cache, sin_cache) + caches:
        if t is not None and t.dtype != ref.dtype:
            raise ValueError("all tensors share the query's dtype")
    if kv8:
        if k_scale is None or v_scale is None:
            raise ValueError("k_scale and v_scale go together")
        if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
            raise ValueError("fp8 caches hold uint8 e4m3 codes")
        for t in (k_scale, v_scale):
            if t.dtype != torch.float32 or t.numel() != hk * d:
                raise ValueError("scales are float32 [Hk, D]")
    if (cos_cache is None) != (sin_cache is None):
        raise ValueError("cos_cache and sin_cache go together")
    max_pos, rdim = (0, 0) if cos_cache is None else (cos_cache.shape[0],
                                                       2 * cos_cache.shape[1])
    if sin_cache is not None and tuple(sin_cache.shape) != tuple(cos_cache.shape):
        raise ValueError("cos_cache and sin_cache shapes differ")
    if not write_q:
        q_out = None
    elif q_out is None:
        q_out = _alloc_on(stream, query, (T, num_heads, d), query.dtype)
    elif q_out.numel() != T * num_heads * d or q_out.dtype != query.dtype:
        raise ValueError("q_out must be [T, Hq, D] of the query's dtype")
    opt = lambda t, n: None if t is None else _dev(t, n)  # noqa: E731
    common = (opt(query, "query"), opt(key, "key"), opt(value, "value"),
              opt(cos_cache, "cos_cache"), opt(sin_cache, "sin_cache"), max_pos, rdim,
              1 if interleaved else 0, _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
              _dev(seqlens_kv, "seqlens_kv", torch.int32),
              _dev(block_table, "block_table", torch.int32))
    tail = (opt(q_out, "q_out"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), B, T, MB, nb,
            num_heads, hk, d, bs, _dtype_code(ref), _stream_ptr(ref, stream))
    if kv8:
        check(lib().pa_rotary_scatter_kv_fp8(*common, _dev(k_scale, "k_scale"),
                                             _dev(v_scale, "v_scale"), *tail))
    else:
        check(lib().pa_rotary_scatter_kv(*common, *tail))
    return q_out


def pa_rotary_scatter_kv(query, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache,
                         num_heads, num_kv_heads, key=None, value=None, cos_cache=None,
                         sin_cache=None, interleaved=False, q_out=None, stream=None,
                         write_q=True):
    """Split packed QKV (``key``/``value`` None: ``query`` is [T, Hq + 2 Hk, D]
    or [T, (Hq + 2 Hk) * D]), rotate Q and K at each token's KV position
    with ``cos_cache``/``sin_cache`` [max_position, rotary_dim / 2] (None: no
    rotation), write K/V into the caches at the block table's slots and
    return the (rotated) Q [T, Hq, D].  ``write_q=False``: Q is not written
    (returns None); pa_attention_rope rotates it as it loads it.  ``query``
    may then be None when ``key``/``value`` are given (K/V only)."""
    return _rotary(query, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, num_heads,
                   num_kv_heads, key, value, cos_cache, sin_cache, interleaved, q_out, stream,
                   write_q)


def pa_rotary_scatter_kv_fp8(query, cu_seqlens_q, seqlens_kv, block_table, k_scale, v_scale,
                             k_cache, v_cache, num_heads, num_kv_heads, key=None, value=None,
                             cos_cache=None, sin_cache=None, interleaved=False, q_out=None,
                             stream=None, write_q=True):
    """pa_rotary_scatter_kv into fp8 (uint8 e4m3) caches with float32
    per-channel scales [Hk, D]: the codes pa_scatter_kv_fp8 writes for the
    rotated rows."""
    return _rotary(query, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, num_heads,
                   num_kv_heads, key, value, cos_cache, sin_cache, interleaved, q_out, stream,
                   write_q, k_scale=k_scale, v_scale=v_scale)


def pa_attention_workspace_size(num_seqs, num_tokens, max_blocks_per_seq, num_heads,
                                num_kv_heads, head_size, block_size):
    """Bytes of device workspace pa_attention needs (0 for invalid sizes)."""
    return int(lib().pa_attention_workspace_size(num_seqs, num_tokens, max_blocks_per_seq,
                                                 num_heads, num_kv_heads, head_size, block_size))


def pa_attention(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, scale,
                 num_heads, num_kv_heads, out=None, workspace=None, stream=None, softcap=0.0,
                 local_window_size=0):
    """Paged causal GQA attention.

    q [T, Hq, D] (or [T, Hq*D]); cu_seqlens_q int32 [B+1]; seqlens_kv int32
    [B]; block_table int32 [B, MB]; caches [NB, bs, Hk, D].  Returns out
    [T, Hq, D].  ``workspace`` is a uint8 GPU tensor of at least
    pa_attention_workspace_size(...) bytes; one is allocated if omitted.
    ``softcap`` c > 0 caps scaled scores as c tanh(x / c);
    ``local_window_size`` W > 0 limits each row to its last W keys.
    """
    import torch
    T = q.shape[0]
    d = k_cache.shape[-1]
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = seqlens_kv.shape[0]
    MB = block_table.shape[1]
    if q.numel() != T * num_heads * d or cu_seqlens_q.shape != (B + 1,) \
            or block_table.shape[0] != B or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or k_cache.shape[2] != num_kv_heads:
        raise ValueError("inconsistent shapes")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and caches must share one dtype")
    if out is None:
        out = _alloc_on(stream, q, (T, num_heads, d), q.dtype)
    elif out.numel() != q.numel() or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = pa_attention_workspace_size(B, T, MB, num_heads, num_kv_heads, d, bs)
    if workspace is None:
        workspace = _alloc_on(stream, q, (max(need, 256),), torch.uint8)
    check(lib().pa_attention(
        _dev(q, "q"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(out, "out"), B, T, MB, nb,
        float(scale), float(softcap), int(local_window_size), num_heads, num_kv_heads, d, bs,
        _dtype_code(q),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream_ptr(q, stream)))
    return out


def pa_attention_rope(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, scale,
                      num_heads, num_kv_heads, cos_cache=None, sin_cache=None, interleaved=False,
                      out=None, workspace=None, stream=None, softcap=0.0, local_window_size=0):
    """pa_attention with Q read from rows of [T, H', D] (H' >= Hq; packed QKV
    rows [T, Hq + 2 Hk, D] as given to pa_rotary_scatter_kv) and rotated as
    it is loaded with ``cos_cache``/``sin_cache`` [max_position,
    rotary_dim / 2] at each token's position (None: no rotation).  Returns
    out [T, Hq, D], bitwise pa_attention on pa_rotary_scatter_kv's Q."""
    import torch
    T = q.shape[0]
    d = k_cache.shape[-1]
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = seqlens_kv.shape[0]
    MB = block_table.shape[1]
    if q.numel() % (T * d) != 0 or q.numel() // (T * d) < num_heads \
            or cu_seqlens_q.shape != (B + 1,) or block_table.shape[0] != B \
            or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[2] != num_kv_heads:
        raise ValueError("inconsistent shapes")
    row = q.numel() // T   # elements per token row
    for t in (k_cache, v_cache, cos_cache, sin_cache):
        if t is not None and t.dtype != q.dtype:
            raise ValueError("all tensors share q's dtype")
    if (cos_cache is None) != (sin_cache is None):
        raise ValueError("cos_cache and sin_cache go together")
    if sin_cache is not None and tuple(sin_cache.shape) != tuple(cos_cache.shape):
        raise ValueError("cos_cache and sin_cache shapes differ")
    max_pos, rdim = (0, 0) if cos_cache is None else (cos_cache.shape[0],
                                                       2 * cos_cache.shape[1])
    if out is None:
        out = _alloc_on(stream, q, (T, num_heads, d), q.dtype)
    elif out.numel() != T * num_heads * d or out.dtype != q.dtype:
        raise ValueError("out must be [T, Hq, D] of q's dtype")
    need = pa_attention_workspace_size(B, T, MB, num_heads, num_kv_heads, d, bs)
    if workspace is None:
        workspace = _alloc_on(stream, q, (max(need, 256),), torch.uint8)
    opt = lambda t, n: None if t is None else _dev(t, n)  # noqa: E731
    check(lib().pa_attention_rope(
        _dev(q, "q"), row, opt(cos_cache, "cos_cache"), opt(sin_cache, "sin_cache"), max_pos,
        rdim, 1 if interleaved else 0, _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(out, "out"), B, T, MB, nb,
        float(scale), float(softcap), int(local_window_size), num_heads, num_kv_heads, d, bs,
        _dtype_code(q), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)))
    return out


def pa_attention_noalloc(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, scale,
                         num_heads, num_kv_heads, out, stream=None, softcap=0.0,
                         local_window_size=0):
    """pa_attention with the library's fixed device scratch instead of a
    workspace: nothing is allocated here or in the library.  ``out`` (the
    caller's [T, Hq, D] tensor) is required for the same reason.  Calls
    that overlap on one GPU share that scratch and must not run
    concurrently."""
    import torch
    T = q.shape[0]
    d = k_cache.shape[-1]
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = seqlens_kv.shape[0]
    MB = block_table.shape[1]
    if q.numel() != T * num_heads * d or cu_seqlens_q.shape != (B + 1,) \
            or block_table.shape[0] != B or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or k_cache.shape[2] != num_kv_heads:
        raise ValueError("inconsistent shapes")
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("q and caches must share one dtype")
    if out is None or out.numel() != q.numel() or out.dtype != q.dtype:
        raise ValueError("out must be given and match q")
    check(lib().pa_attention_noalloc(
        _dev(q, "q"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(out, "out"), B, T, MB, nb,
        float(scale), float(softcap), int(local_window_size), num_heads, num_kv_heads, d, bs,
        _dtype_code(q), _stream_ptr(q, stream)))
    return out


def pa_scatter_kv_fp8(k_new, v_new, slot_mapping, k_scale, v_scale, k_cache, v_cache,
                      stream=None):
    """Quantize new K/V rows [T, Hk, D] (fp16/bf16) into fp8 (e4m3) caches
    [NB, bs, Hk, D] (uint8 codes) with float32 per-channel scales [Hk, D], at
    int32 ``slot_mapping`` [T] (negative = skip), in place."""
    import torch
    T, hk, d = k_new.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    if tuple(v_new.shape) != (T, hk, d) or tuple(k_cache.shape) != (nb, bs, hk, d) \
            or tuple(v_cache.shape) != (nb, bs, hk, d) or slot_mapping.shape != (T,) \
            or tuple(k_scale.shape) != (hk, d) or tuple(v_scale.shape) != (hk, d):
        raise ValueError("inconsistent shapes")
    if k_new.dtype != v_new.dtype or k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("K/V share one 16-bit dtype; the caches hold uint8 codes")
    check(lib().pa_scatter_kv_fp8(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(slot_mapping, "slot_mapping", torch.int32),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), T, nb, hk, d, bs,
        _dtype_code(k_new), _stream_ptr(k_cache, stream)))


def pa_scatter_kv_paged_fp8(k_new, v_new, cu_seqlens_q, seqlens_kv, block_table, k_scale,
                            v_scale, k_cache, v_cache, stream=None):
    """pa_scatter_kv_fp8 with the slots derived on the GPU as
    pa_scatter_kv_paged derives them: token t of sequence b is quantized
    into KV position past_b + (t - cu[b]) of b's block-table row."""
    import torch
    T, hk, d = k_new.shape
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = cu_seqlens_q.shape[0] - 1
    if tuple(v_new.shape) != (T, hk, d) or tuple(k_cache.shape) != (nb, bs, hk, d) \
            or tuple(v_cache.shape) != (nb, bs, hk, d) or seqlens_kv.shape != (B,) \
            or block_table.dim() != 2 or block_table.shape[0] != B \
            or tuple(k_scale.shape) != (hk, d) or tuple(v_scale.shape) != (hk, d):
        raise ValueError("inconsistent shapes")
    if k_new.dtype != v_new.dtype or k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("K/V share one 16-bit dtype; the caches hold uint8 codes")
    check(lib().pa_scatter_kv_paged_fp8(
        _dev(k_new, "k_new"), _dev(v_new, "v_new"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), B, T, block_table.shape[1], nb, hk, d,
        bs, _dtype_code(k_new), _stream_ptr(k_cache, stream)))


def pa_attention_fp8(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, k_scale,
                     v_scale, scale, num_heads, num_kv_heads, max_q_len, out=None,
                     workspace=None, stream=None, softcap=0.0, local_window_size=0):
    """pa_attention over fp8 (e4m3) caches [NB, bs, Hk, D] (uint8 codes) with
    float32 per-channel scales [Hk, D], for batches whose every q_len * G is
    at most 16 (``max_q_len`` is a host-side bound of q_len).  ``softcap``
    and ``local_window_size`` as for pa_attention."""
    import torch
    T = q.shape[0]
    d = k_cache.shape[-1]
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = seqlens_kv.shape[0]
    MB = block_table.shape[1]
    if q.numel() != T * num_heads * d or cu_seqlens_q.shape != (B + 1,) \
            or block_table.shape[0] != B or tuple(v_cache.shape) != tuple(k_cache.shape) \
            or k_cache.shape[2] != num_kv_heads or tuple(k_scale.shape) != (num_kv_heads, d) \
            or tuple(v_scale.shape) != (num_kv_heads, d):
        raise ValueError("inconsistent shapes")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches hold uint8 codes")
    if out is None:
        out = _alloc_on(stream, q, (T, num_heads, d), q.dtype)
    elif out.numel() != q.numel() or out.dtype != q.dtype:
        raise ValueError("out must match q")
    need = pa_attention_workspace_size(B, T, MB, num_heads, num_kv_heads, d, bs)
    if workspace is None:
        workspace = _alloc_on(stream, q, (max(need, 256),), torch.uint8)
    check(lib().pa_attention_fp8(
        _dev(q, "q"), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(out, "out"), B, T, int(max_q_len), MB, nb, float(scale), float(softcap),
        int(local_window_size), num_heads, num_kv_heads, d, bs, _dtype_code(q), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream_ptr(q, stream)))
    return out


def pa_attention_rope_fp8(q, cu_seqlens_q, seqlens_kv, block_table, k_cache, v_cache, k_scale,
                          v_scale, scale, num_heads, num_kv_heads, max_q_len, cos_cache=None,
                          sin_cache=None, interleaved=False, out=None, workspace=None,
                          stream=None, softcap=0.0, local_window_size=0):
    """pa_attention_fp8 with Q read from rows of [T, H', D] (H' >= Hq; packed
    QKV rows [T, Hq + 2 Hk, D]) and rotated as it is loaded, as in
    pa_attention_rope.  Returns out [T, Hq, D], bitwise pa_attention_fp8 on
    pa_rotary_scatter_kv_fp8's Q."""
    import torch
    T = q.shape[0]
    d = k_cache.shape[-1]
    nb, bs = k_cache.shape[0], k_cache.shape[1]
    B = seqlens_kv.shape[0]
    MB = block_table.shape[1]
    if q.numel() % (T * d) != 0 or q.numel() // (T * d) < num_heads \
            or cu_seqlens_q.shape != (B + 1,) or block_table.shape[0] != B \
            or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[2] != num_kv_heads \
            or tuple(k_scale.shape) != (num_kv_heads, d) \
            or tuple(v_scale.shape) != (num_kv_heads, d):
        raise ValueError("inconsistent shapes")
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise ValueError("fp8 caches hold uint8 codes")
    row = q.numel() // T   # elements per token row
    for t in (cos_cache, sin_cache):
        if t is not None and t.dtype != q.dtype:
            raise ValueError("the rotary tables share q's dtype")
    if (cos_cache is None) != (sin_cache is None):
        raise ValueError("cos_cache and sin_cache go together")
    if sin_cache is not None and tuple(sin_cache.shape) != tuple(cos_cache.shape):
        raise ValueError("cos_cache and sin_cache shapes differ")
    max_pos, rdim = (0, 0) if cos_cache is None else (cos_cache.shape[0],
                                                       2 * cos_cache.shape[1])
    if out is None:
        out = _alloc_on(stream, q, (T, num_heads, d), q.dtype)
    elif out.numel() != T * num_heads * d or out.dtype != q.dtype:
        raise ValueError("out must be [T, Hq, D] of q's dtype")
    need = pa_attention_workspace_size(B, T, MB, num_heads, num_kv_heads, d, bs)
    if workspace is None:
        workspace = _alloc_on(stream, q, (max(need, 256),), torch.uint8)
    opt = lambda t, n: None if t is None else _dev(t, n)  # noqa: E731
    check(lib().pa_attention_rope_fp8(
        _dev(q, "q"), row, opt(cos_cache, "cos_cache"), opt(sin_cache, "sin_cache"), max_pos,
        rdim, 1 if interleaved else 0, _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32),
        _dev(seqlens_kv, "seqlens_kv", torch.int32), _dev(block_table, "block_table", torch.int32),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
        _dev(k_scale, "k_scale", torch.float32), _dev(v_scale, "v_scale", torch.float32),
        _dev(out, "out"), B, T, int(max_q_len), MB, nb, float(scale), float(softcap),
        int(local_window_size), num_heads, num_kv_heads, d, bs, _dtype_code(q),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream_ptr(q, stream)))
    return out


def pa_validate_metadata(cu_seqlens_q, seqlens_kv, block_table, num_blocks, block_size,
                         slot_mapping=None, num_tokens=None, stream=None):
    """Debug check of device metadata; returns the violation bit mask
    (0 = valid).  Synchronises the stream."""
    import torch
    B = seqlens_kv.shape[0]
    T = int(num_tokens if num_tokens is not None else
            (slot_mapping.shape[0] if slot_mapping is not None else 0))
    v = ctypes.c_uint32(0)
    check(lib().pa_validate_metadata(
        _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(seqlens_kv, "seqlens_kv", torch.int32),
        _dev(block_table, "block_table", torch.int32),
        _dev(slot_mapping, "slot_mapping", torch.int32) if slot_mapping is not None else None,
        B, T, block_table.shape[1], num_blocks, block_size, ctypes.byref(v),
        _stream_ptr(seqlens_kv, stream)))
    return int(v.value)


def profile_enable(on=True):
    check(lib().pa_profile_enable(1 if on else 0))


def profile_select(kinds=None):
    """Time only the kernel kinds named in ``kinds`` (names from
    PROFILE_KINDS); None: every kind."""
    if kinds is None:
        mask = (1 << len(PROFILE_KINDS)) - 1
    else:
        unknown = set(kinds) - set(PROFILE_KINDS)
        if unknown:
            raise ValueError(f"unknown kernel kinds {sorted(unknown)}")
        mask = sum(1 << PROFILE_KINDS.index(k) for k in kinds)
    check(lib().pa_profile_select(mask))


def profile_read():
    """{kernel kind: (total ms, launches)} since the last read."""
    n = len(PROFILE_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    check(lib().pa_profile_read(ms, cnt, n))
    return {k: (ms[i], cnt[i]) for i, k in enumerate(PROFILE_KINDS)}
