"""Exact softmax attention on MI355X (gfx950): a thin Python binding of libattn.so.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/attn.h``; this module only marshals torch tensors into
pointers, sizes and the current HIP stream, and turns non-zero status codes
into exceptions.  torch provides device memory and streams, nothing else.

Entry points (same names as the C ABI):

* ``prefill_fwd(q, k, v, causal, scale)`` -- ``attn_prefill_fwd``
* ``decode_splitk(q, k_cache, v_cache, kv_lens, num_splits, scale)`` -- ``attn_decode_splitk``
* ``merge_partials(part_m, part_l, part_o, out_dtype)`` -- ``attn_merge_partials``
* ``decode(...)`` -- the two decode calls back to back on one stream
* ``decode_num_splits``, ``decode_chunk_len``, ``decode_workspace_bytes`` -- host helpers
"""

from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib
from ._lib import ATTN_BF16, ATTN_F16, AttnError  # noqa: F401

__all__ = ["prefill_fwd", "decode_splitk", "merge_partials", "decode", "decode_num_splits", "decode_chunk_len",
           "decode_workspace_bytes", "AttnError"]

_DTYPES = {torch.bfloat16: ATTN_BF16, torch.float16: ATTN_F16}


def _lib_handle():
    return _lib.load()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported element type {t.dtype}; expected bfloat16 or float16")
    return _DTYPES[t.dtype]


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _scale(scale: Optional[float], d: int) -> float:
    return float(1.0 / math.sqrt(d)) if scale is None else float(scale)


def prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact attention of ``q: [B, Hq, N, d]`` over ``k, v: [B, Hkv, N, d]``; returns ``[B, Hq, N, d]``."""
    lib = _lib_handle()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, hq, n, d = q.shape
    if k.shape[0] != B or k.shape[2] != n or k.shape[3] != d or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v disagree in batch, length, head dim or dtype")
    if out is None:
        out = torch.empty_like(q)
    st = lib.attn_prefill_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dtype_code(q), B, hq,
                              k.shape[1], n, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _lib.check("attn_prefill_fwd", st)
    return out


def decode_num_splits(batch: int, hkv: int, max_kv_len: int) -> int:
    return int(_lib_handle().attn_decode_num_splits(batch, hkv, max_kv_len))


def decode_chunk_len(max_kv_len: int, num_splits: int) -> int:
    return int(_lib_handle().attn_decode_chunk_len(max_kv_len, num_splits))


def decode_workspace_bytes(batch: int, hq: int, d: int, num_splits: int) -> int:
    return int(_lib_handle().attn_decode_workspace_bytes(batch, hq, d, num_splits))


def decode_splitk(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor,
                  num_splits: Optional[int] = None, scale: Optional[float] = None, partials=None):
    """Partial states ``(m, l, o)`` of each split: ``m, l: [B, Hq, S]``, ``o: [B, Hq, S, d]`` fp32."""
    lib = _lib_handle()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B, Hq, d] and caches [B, Hkv, Lmax, d]")
    B, hq, d = q.shape
    _, hkv, L, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches disagree in batch, head dim or dtype")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
        raise ValueError("kv_lens must be an int32 device tensor with one entry per sequence")
    S = decode_num_splits(B, hkv, L) if num_splits is None else int(num_splits)
    if partials is None:
        pm = torch.empty((B, hq, S), dtype=torch.float32, device=q.device)
        pl = torch.empty((B, hq, S), dtype=torch.float32, device=q.device)
        po = torch.empty((B, hq, S, d), dtype=torch.float32, device=q.device)
    else:
        pm, pl, po = partials
    st = lib.attn_decode_splitk(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(kv_lens, "kv_lens"), L, _dtype_code(q), B, hq, hkv, d, _scale(scale, d), S,
                                _dev(pm, "part_m"), _dev(pl, "part_l"), _dev(po, "part_o"), _stream(q))
    _lib.check("attn_decode_splitk", st)
    return pm, pl, po


def merge_partials(part_m: torch.Tensor, part_l: torch.Tensor, part_o: torch.Tensor,
                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Merge ``[B, Hq, S]`` / ``[B, Hq, S, d]`` fp32 partials into ``[B, Hq, d]`` of ``out_dtype``."""
    lib = _lib_handle()
    B, hq, S, d = part_o.shape
    if part_m.shape != (B, hq, S) or part_l.shape != (B, hq, S):
        raise ValueError("partial shapes disagree")
    if any(t.dtype != torch.float32 for t in (part_m, part_l, part_o)):
        raise TypeError("partials must be float32")
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype, device=part_o.device)
    st = lib.attn_merge_partials(_dev(part_m, "part_m"), _dev(part_l, "part_l"), _dev(part_o, "part_o"), B, hq, d,
                                 S, _dev(out, "out"), _DTYPES[out.dtype], _stream(part_o))
    _lib.check("attn_merge_partials", st)
    return out


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor,
           num_splits: Optional[int] = None, scale: Optional[float] = None, partials=None) -> torch.Tensor:
    """Single-query decode: split-K partials then their merge, on the current stream."""
    pm, pl, po = decode_splitk(q, k_cache, v_cache, kv_lens, num_splits, scale, partials)
    return merge_partials(pm, pl, po, q.dtype)
