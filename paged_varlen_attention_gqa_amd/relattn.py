"""Thin Python binding of librelattn.so (ctypes).

Argument marshalling only: every step of the attention runs in the HIP
kernels behind the C ABI (include/rel_attn.h). PyTorch provides device memory
and the current HIP stream. There is no fallback: if the library is missing
or a call fails, an exception is raised.

The keyword arguments follow the documented ``inkling_fa4_rel_attention``
signature (docs.vllm.ai API page of
``vllm.models.inkling.nvidia.ops.fa4_rel_attention``).
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "librelattn.so")

FP32 = 0
BF16 = 1
MAX_SPLITS = 512

_lib = None


class RelAttnError(RuntimeError):
    pass


def load_library() -> ctypes.CDLL:
    """Load librelattn.so (built by ``paged_varlen_attention_gqa_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RelAttnError(
            f"{LIB_PATH} is not built; run `python -m paged_varlen_attention_gqa_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_int, c_size, c_vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p
    lib.rel_attn_num_splits.argtypes = [c_int] * 6
    lib.rel_attn_num_splits.restype = c_int
    lib.rel_attn_workspace_bytes.argtypes = [c_int] * 4
    lib.rel_attn_workspace_bytes.restype = c_size
    lib.rel_attn_strerror.argtypes = [c_int]
    lib.rel_attn_strerror.restype = ctypes.c_char_p
    lib.rel_attn_fwd.argtypes = (
        [c_vp] * 8                      # q, k, v, block_table, cache_seqlens, cu_q, rel, out
        + [c_int] * 11                  # dtype .. rel_extent
        + [ctypes.c_float]              # softmax_scale
        + [c_int] * 4                   # causal, window_left, window_right, num_splits
        + [c_vp, c_size, ctypes.POINTER(c_size), c_vp]
    )
    lib.rel_attn_fwd.restype = c_int
    lib.rel_attn_fwd_splits.argtypes = lib.rel_attn_fwd.argtypes
    lib.rel_attn_fwd_splits.restype = c_int
    lib.rel_attn_fwd_lse.argtypes = [c_vp] * 9 + lib.rel_attn_fwd.argtypes[8:]  # + lse after out
    lib.rel_attn_fwd_lse.restype = c_int
    lib.rel_attn_combine.argtypes = [c_vp, c_size, c_vp] + [c_int] * 5 + [c_vp]
    lib.rel_attn_combine.restype = c_int
    lib.rel_attn_fwd_noalloc.argtypes = lib.rel_attn_fwd.argtypes[:24] + [c_vp]  # no workspace arguments
    lib.rel_attn_fwd_noalloc.restype = c_int
    lib.rel_attn_noalloc_scratch_bytes.argtypes = []
    lib.rel_attn_noalloc_scratch_bytes.restype = c_size
    _lib = lib
    return lib


def rel_attn_strerror(code: int) -> str:
    return load_library().rel_attn_strerror(int(code)).decode()


def rel_attn_num_splits(*, is_local: bool, batch_size: int, max_query_len: int, num_heads: int,
                        num_kv_heads: int, max_kv_len: int) -> int:
    """Split-KV count for a call of this shape (host only); see include/rel_attn.h."""
    r = load_library().rel_attn_num_splits(int(bool(is_local)), int(batch_size), int(max_query_len),
                                           int(num_heads), int(num_kv_heads), int(max_kv_len))
    if r < 0:
        raise RelAttnError(f"rel_attn_num_splits: {rel_attn_strerror(r)}")
    return r


def rel_attn_workspace_bytes(num_splits: int, num_tokens: int, num_heads: int, head_dim: int) -> int:
    return int(load_library().rel_attn_workspace_bytes(int(num_splits), int(num_tokens),
                                                       int(num_heads), int(head_dim)))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check_dev(name, t, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")


def _attention_call(entry: str, q, key_cache, value_cache, *, block_table, cache_seqlens,
                    cu_seqlens_q, max_seqlen_q, softmax_scale, causal, window_size, rel_extent,
                    rel_logits, num_splits, out, workspace, max_kv_len, lse=None):
    lib = load_library()
    if q.dtype == torch.bfloat16:
        dt = BF16
    elif q.dtype == torch.float32:
        dt = FP32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for name, t in (("q", q), ("key_cache", key_cache), ("value_cache", value_cache)):
        _check_dev(name, t, q.dtype)
    for name, t in (("block_table", block_table), ("cache_seqlens", cache_seqlens),
                    ("cu_seqlens_q", cu_seqlens_q)):
        _check_dev(name, t, torch.int32)
    if rel_extent > 0:
        _check_dev("rel_logits", rel_logits, q.dtype)
    T, H, D = q.shape
    NB, BS, HKV, D2 = key_cache.shape
    if D2 != D or tuple(value_cache.shape) != tuple(key_cache.shape):
        raise ValueError("key_cache / value_cache shape mismatch")
    B = cache_seqlens.shape[0]
    if cu_seqlens_q.shape[0] != B + 1 or block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("metadata shape mismatch")
    if rel_extent > 0 and tuple(rel_logits.shape) != (T, H, rel_extent):
        raise ValueError(f"rel_logits must be {(T, H, rel_extent)}, got {tuple(rel_logits.shape)}")
    wl, wr = (int(window_size[0]), int(window_size[1]))
    if num_splits is None:
        mk = max_kv_len if max_kv_len is not None else block_table.shape[1] * BS
        num_splits = rel_attn_num_splits(is_local=(wl >= 0 or wr >= 0), batch_size=max(B, 1),
                                         max_query_len=max(int(max_seqlen_q), 1), num_heads=H,
                                         num_kv_heads=HKV, max_kv_len=mk)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_dev("out", out, q.dtype)
        if out.shape != q.shape:
            raise ValueError("out must have the shape of q")
    with_lse = entry == "rel_attn_fwd_lse"
    if with_lse:
        if lse is None:
            lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
        else:
            _check_dev("lse", lse, torch.float32)
            if tuple(lse.shape) != (T, H):
                raise ValueError(f"lse must be {(T, H)}, got {tuple(lse.shape)}")
    need = rel_attn_workspace_bytes(max(num_splits, 2) if with_lse else num_splits, T, H, D)
    if entry == "rel_attn_fwd_noalloc":
        need = 0  # the library's own scratch array holds the partials
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        else:
            _check_dev("workspace", workspace)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if entry == "rel_attn_fwd_noalloc":
        rc = lib.rel_attn_fwd_noalloc(
            _ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(block_table), _ptr(cache_seqlens),
            _ptr(cu_seqlens_q), _ptr(rel_logits if rel_extent > 0 else None), _ptr(out),
            dt, T, B, int(max_seqlen_q), block_table.shape[1], H, HKV, D, NB, BS, int(rel_extent),
            float(softmax_scale), int(bool(causal)), wl, wr, int(num_splits), ctypes.c_void_p(stream))
        if rc != 0:
            raise RelAttnError(f"{entry}: {rel_attn_strerror(rc)} (code {rc})")
        return out, None, num_splits
    lse_arg = [_ptr(lse)] if with_lse else []
    rc = getattr(lib, entry)(
        _ptr(q), _ptr(key_cache), _ptr(value_cache), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(cu_seqlens_q), _ptr(rel_logits if rel_extent > 0 else None), _ptr(out), *lse_arg,
        dt, T, B, int(max_seqlen_q), block_table.shape[1], H, HKV, D, NB, BS, int(rel_extent),
        float(softmax_scale), int(bool(causal)), wl, wr, int(num_splits),
        _ptr(workspace) if need > 0 else ctypes.c_void_p(0), ws_bytes, None,
        ctypes.c_void_p(stream))
    if rc != 0:
        raise RelAttnError(f"{entry}: {rel_attn_strerror(rc)} (code {rc})")
    if with_lse:
        return out, lse, num_splits
    return out, workspace, num_splits


def rel_attn_fwd(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor, *,
                 block_table: torch.Tensor, cache_seqlens: torch.Tensor, cu_seqlens_q: torch.Tensor,
                 max_seqlen_q: int, softmax_scale: float, causal: bool, window_size=(-1, -1),
                 rel_extent: int, rel_logits: torch.Tensor | None, num_splits: int | None = None,
                 out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                 max_kv_len: int | None = None, return_lse: bool = False,
                 lse: torch.Tensor | None = None):
    """Paged varlen GQA attention with the per-token relative bias; returns ``out``,
    or ``(out, lse)`` with ``return_lse=True`` (``lse`` (num_tokens, num_heads)
    float32, natural log, -inf for rows without visible keys; the call then
    runs split, at least 2 pieces).

    ``num_splits=None`` asks :func:`rel_attn_num_splits`, with ``max_kv_len``
    defaulting to the page-table capacity (``block_table.shape[1] *
    block_size``), so no device value is read on the host.
    """
    res, extra, _ = _attention_call(
        "rel_attn_fwd_lse" if return_lse else "rel_attn_fwd", q, key_cache, value_cache,
        block_table=block_table, cache_seqlens=cache_seqlens, cu_seqlens_q=cu_seqlens_q,
        max_seqlen_q=max_seqlen_q, softmax_scale=softmax_scale, causal=causal,
        window_size=window_size, rel_extent=rel_extent, rel_logits=rel_logits,
        num_splits=num_splits, out=out, workspace=workspace, max_kv_len=max_kv_len, lse=lse)
    return (res, extra) if return_lse else res


def rel_attn_fwd_splits(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor, *,
                        block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                        causal: bool, window_size=(-1, -1), rel_extent: int,
                        rel_logits: torch.Tensor | None, num_splits: int | None = None,
                        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                        max_kv_len: int | None = None):
    """The attention stage alone; returns ``(out, workspace, num_splits)``.

    With one split ``out`` holds the result. With more, ``out`` is untouched
    and ``workspace`` holds the per-split partial outputs and log-sum-exps
    (layout in include/rel_attn.h); :func:`rel_attn_combine` merges them.
    """
    return _attention_call(
        "rel_attn_fwd_splits", q, key_cache, value_cache, block_table=block_table,
        cache_seqlens=cache_seqlens, cu_seqlens_q=cu_seqlens_q, max_seqlen_q=max_seqlen_q,
        softmax_scale=softmax_scale, causal=causal, window_size=window_size, rel_extent=rel_extent,
        rel_logits=rel_logits, num_splits=num_splits, out=out, workspace=workspace,
        max_kv_len=max_kv_len)


def rel_attn_fwd_noalloc(q: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor, *,
                         block_table: torch.Tensor, cache_seqlens: torch.Tensor,
                         cu_seqlens_q: torch.Tensor, max_seqlen_q: int, softmax_scale: float,
                         causal: bool, window_size=(-1, -1), rel_extent: int,
                         rel_logits: torch.Tensor | None, num_splits: int | None = None,
                         out: torch.Tensor | None = None, max_kv_len: int | None = None):
    """:func:`rel_attn_fwd` through the entry point that allocates nothing: the
    split partials go to the library's static scratch array (at most
    :func:`rel_attn_noalloc_scratch_bytes` bytes). Pass ``out`` to keep the
    call free of allocations on the Python side too."""
    res, _, _ = _attention_call(
        "rel_attn_fwd_noalloc", q, key_cache, value_cache, block_table=block_table,
        cache_seqlens=cache_seqlens, cu_seqlens_q=cu_seqlens_q, max_seqlen_q=max_seqlen_q,
        softmax_scale=softmax_scale, causal=causal, window_size=window_size, rel_extent=rel_extent,
        rel_logits=rel_logits, num_splits=num_splits, out=out, workspace=None, max_kv_len=max_kv_len)
    return res


def rel_attn_noalloc_scratch_bytes() -> int:
    """Size of the static scratch array behind :func:`rel_attn_fwd_noalloc`."""
    return int(load_library().rel_attn_noalloc_scratch_bytes())


def split_partials(workspace: torch.Tensor, num_splits: int, num_tokens: int, num_heads: int,
                   head_dim: int):
    """Views ``(o [splits, T, H, D], lse [splits, T, H])`` of a split workspace (fp32)."""
    n_o = num_splits * num_tokens * num_heads * head_dim
    f = workspace.view(torch.float32)
    o = f[:n_o].view(num_splits, num_tokens, num_heads, head_dim)
    lse = f[n_o:n_o + num_splits * num_tokens * num_heads].view(num_splits, num_tokens, num_heads)
    return o, lse


def rel_attn_combine(workspace: torch.Tensor, out: torch.Tensor, num_splits: int) -> torch.Tensor:
    """Merge the partials of :func:`rel_attn_fwd_splits` into ``out`` [T, H, D]; returns ``out``."""
    lib = load_library()
    _check_dev("workspace", workspace)
    _check_dev("out", out)
    if out.dtype == torch.bfloat16:
        dt = BF16
    elif out.dtype == torch.float32:
        dt = FP32
    else:
        raise ValueError(f"unsupported dtype {out.dtype}")
    T, H, D = out.shape
    stream = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib.rel_attn_combine(_ptr(workspace), workspace.numel() * workspace.element_size(),
                              _ptr(out), dt, T, H, D, int(num_splits), ctypes.c_void_p(stream))
    if rc != 0:
        raise RelAttnError(f"rel_attn_combine: {rel_attn_strerror(rc)} (code {rc})")
    return out
