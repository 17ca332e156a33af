"""Exact softmax attention on MI355X (gfx950): a thin Python binding of libattn.so.

Every step of the computation runs in the HIP kernels behind the C ABI
declared in ``include/attn.h``; this module only marshals torch tensors into
pointers, sizes and the current HIP stream, and turns non-zero status codes
into exceptions.  torch provides device memory and streams, nothing else.

Entry points (same names as the C ABI):

* ``prefill_fwd(q, k, v, causal, scale)`` -- ``attn_prefill_fwd``
* ``prefill_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, causal, scale)`` --
  ``attn_prefill_varlen_fwd``
* ``decode_splitk(q, k_cache, v_cache, kv_lens, num_splits, scale)`` -- ``attn_decode_splitk``
* ``decode_splitk_paged(q, k_pages, v_pages, block_table, kv_lens, num_splits, scale)`` --
  ``attn_decode_splitk_paged``
* ``decode_splitk_q4(q, k_codes, k_scales, v_codes, v_scales, kv_lens, rotated, num_splits, scale)`` --
  ``attn_decode_splitk_q4``
* ``decode_splitk_q4_paged(q, k_codes, k_scales, v_codes, v_scales, block_table, kv_lens, rotated, num_splits,
  scale)`` -- ``attn_decode_splitk_q4_paged``
* ``kv_quantize_q4(x, rotated, out_rows, codes, scales)`` -- ``attn_kv_quantize_q4``
* ``merge_partials(part_m, part_l, part_o, out_dtype)`` -- ``attn_merge_partials``
* ``decode(...)``, ``decode_paged(...)``, ``decode_q4(...)``, ``decode_q4_paged(...)`` -- split-K then merge, back to
  back on one stream
* ``decode_noalloc(q, k_cache, v_cache, kv_lens, num_splits, scale)`` -- ``attn_decode_noalloc``: the same
  split-K and merge with the partial states in the library's fixed scratch array (no workspace)
* ``decode_num_splits``, ``decode_q4_num_splits``, ``decode_chunk_len``, ``decode_workspace_bytes`` -- host helpers
"""

from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib
from ._lib import ATTN_BF16, ATTN_F16, AttnError  # noqa: F401

__all__ = ["prefill_fwd", "prefill_varlen_fwd", "decode_splitk", "decode_splitk_paged", "decode_splitk_q4", "decode_q4",
           "decode_splitk_q4_paged", "decode_q4_paged", "kv_quantize_q4", "merge_partials", "decode", "decode_paged",
           "decode_noalloc", "decode_num_splits", "decode_q4_num_splits", "decode_chunk_len", "decode_workspace_bytes", "AttnError"]

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


def _check(t: torch.Tensor, name: str, shape, dtype: torch.dtype, device: torch.device) -> torch.Tensor:
    """A caller-supplied buffer must be exactly what the kernels will write:
    the kernels trust the sizes they are given, so a wrong one is refused here."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _same_device(ref: torch.Tensor, **tensors) -> None:
    for name, t in tensors.items():
        if t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _partials(partials, B: int, hq: int, S: int, d: int, device: torch.device):
    """The split-K workspace ``(m [B, hq, S], l [B, hq, S], o [B, hq, S, d])``, fp32 on ``device``:
    allocated here when not given, else checked against the split count the call uses."""
    if partials is None:
        return (torch.empty((B, hq, S), dtype=torch.float32, device=device),
                torch.empty((B, hq, S), dtype=torch.float32, device=device),
                torch.empty((B, hq, S, d), dtype=torch.float32, device=device))
    if len(partials) != 3:
        raise ValueError("partials must be a (part_m, part_l, part_o) triple")
    pm, pl, po = partials
    return (_check(pm, "part_m", (B, hq, S), torch.float32, device),
            _check(pl, "part_l", (B, hq, S), torch.float32, device),
            _check(po, "part_o", (B, hq, S, d), torch.float32, device))


def prefill_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                scale: Optional[float] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Exact attention of ``q: [B, Hq, N, d]`` over ``k, v: [B, Hkv, N, d]``; returns ``[B, Hq, N, d]``."""
    lib = _lib_handle()
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B, Hq, N, d] and k, v [B, Hkv, N, d]")
    B, hq, n, d = q.shape
    if k.shape[0] != B or k.shape[2] != n or k.shape[3] != d or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v disagree in batch, length, head dim or dtype")
    _same_device(q, k=k, v=v)
    out = torch.empty_like(q) if out is None else _check(out, "out", q.shape, q.dtype, q.device)
    st = lib.attn_prefill_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), _dtype_code(q), B, hq,
                              k.shape[1], n, d, _scale(scale, d), int(bool(causal)), _stream(q))
    _lib.check("attn_prefill_fwd", st)
    return out


def prefill_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                       cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, causal: bool = False,
                       scale: Optional[float] = None, out: Optional[torch.Tensor] = None, window: int = 0,
                       alibi_slopes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Packed variable-length prefill / append: ``q [total_q, Hq, d]``, ``k, v [total_k, Hkv, d]``,
    ``cu_seqlens_*`` int32 device tensors of ``batch + 1`` offsets; returns ``[total_q, Hq, d]``.
    Queries are bottom-right aligned: query i of a sequence (position p = i + nk - nq) sees keys j <= p when
    causal, and only p - window < j when ``window > 0``; ``alibi_slopes`` (fp32 device ``[Hq]``) adds
    ``-slope·(p - j)`` to each score."""
    lib = _lib_handle()
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("expected q [total_q, Hq, d] and k, v [total_k, Hkv, d]")
    total_q, hq, d = q.shape
    total_k, hkv, dk = k.shape
    if dk != d or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v disagree in head dim or dtype")
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu.dtype != torch.int32 or cu.dim() != 1 or cu.device != q.device:
            raise ValueError(f"{name} must be a 1-D int32 device tensor")
    if cu_seqlens_k.numel() != cu_seqlens_q.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold batch + 1 >= 2 offsets")
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != hq
                                     or alibi_slopes.device != q.device):
        raise ValueError("alibi_slopes must be a float32 device tensor with one slope per query head")
    _same_device(q, k=k, v=v)
    out = torch.empty_like(q) if out is None else _check(out, "out", q.shape, q.dtype, q.device)
    st = lib.attn_prefill_varlen_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                                     _dev(cu_seqlens_q, "cu_seqlens_q"), _dev(cu_seqlens_k, "cu_seqlens_k"), total_q,
                                     total_k, int(max_seqlen_q), int(max_seqlen_k), _dtype_code(q),
                                     cu_seqlens_q.numel() - 1, hq, hkv, d, _scale(scale, d), int(bool(causal)),
                                     int(window), None if alibi_slopes is None else _dev(alibi_slopes, "alibi_slopes"),
                                     _stream(q))
    _lib.check("attn_prefill_varlen_fwd", st)
    return out


def decode_num_splits(batch: int, hkv: int, max_kv_len: int) -> int:
    return int(_lib_handle().attn_decode_num_splits(batch, hkv, max_kv_len))


def decode_q4_num_splits(batch: int, hkv: int, max_kv_len: int) -> int:
    return int(_lib_handle().attn_decode_q4_num_splits(batch, hkv, max_kv_len))


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
    _same_device(q, k_cache=k_cache, v_cache=v_cache)
    S = decode_num_splits(B, hkv, L) if num_splits is None else int(num_splits)
    pm, pl, po = _partials(partials, B, hq, S, d, q.device)
    st = lib.attn_decode_splitk(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(kv_lens, "kv_lens"), L, _dtype_code(q), B, hq, hkv, d, _scale(scale, d), S,
                                _dev(pm, "part_m"), _dev(pl, "part_l"), _dev(po, "part_o"), _stream(q))
    _lib.check("attn_decode_splitk", st)
    return pm, pl, po


def decode_splitk_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                        kv_lens: torch.Tensor, num_splits: Optional[int] = None, scale: Optional[float] = None,
                        partials=None, window: int = 0, alibi_slopes: Optional[torch.Tensor] = None):
    """Partial states over a paged cache: ``k_pages, v_pages: [P, Hkv, page, d]``,
    ``block_table: [B, max_pages]`` int32 (device).  Same outputs as ``decode_splitk``; ``window > 0`` keeps
    only the last ``window`` keys, ``alibi_slopes`` (fp32 device ``[Hq]``) adds ``-slope·(p - j)``."""
    lib = _lib_handle()
    if q.dim() != 3 or k_pages.dim() != 4 or v_pages.shape != k_pages.shape or block_table.dim() != 2:
        raise ValueError("expected q [B, Hq, d], pages [P, Hkv, page, d] and block_table [B, max_pages]")
    B, hq, d = q.shape
    P, hkv, page, dk = k_pages.shape
    if dk != d or k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise ValueError("q and pages disagree in head dim or dtype")
    if block_table.dtype != torch.int32 or block_table.shape[0] != B or block_table.device != q.device:
        raise ValueError("block_table must be an int32 device tensor [B, max_pages]")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
        raise ValueError("kv_lens must be an int32 device tensor with one entry per sequence")
    if alibi_slopes is not None and (alibi_slopes.dtype != torch.float32 or alibi_slopes.numel() != hq
                                     or alibi_slopes.device != q.device):
        raise ValueError("alibi_slopes must be a float32 device tensor with one slope per query head")
    _same_device(q, k_pages=k_pages, v_pages=v_pages)
    max_pages = block_table.shape[1]
    S = decode_num_splits(B, hkv, max_pages * page) if num_splits is None else int(num_splits)
    pm, pl, po = _partials(partials, B, hq, S, d, q.device)
    st = lib.attn_decode_splitk_paged(_dev(q, "q"), _dev(k_pages, "k_pages"), _dev(v_pages, "v_pages"),
                                      _dev(block_table, "block_table"), max_pages, P, page,
                                      _dev(kv_lens, "kv_lens"), _dtype_code(q), B, hq, hkv, d, _scale(scale, d), S,
                                      int(window), None if alibi_slopes is None else _dev(alibi_slopes, "alibi"),
                                      _dev(pm, "part_m"), _dev(pl, "part_l"), _dev(po, "part_o"), _stream(q))
    _lib.check("attn_decode_splitk_paged", st)
    return pm, pl, po


def decode_splitk_q4(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                     v_scales: torch.Tensor, kv_lens: torch.Tensor, rotated: bool, num_splits: Optional[int] = None,
                     scale: Optional[float] = None, partials=None):
    """Partial states over a 4-bit cache: ``k_codes, v_codes: [B, Hkv, Lmax, d/2]`` uint8 (E2M1 pairs),
    ``k_scales, v_scales: [B, Hkv, Lmax]`` fp32; ``rotated``: rows stored in the normalised Hadamard domain."""
    lib = _lib_handle()
    if q.dim() != 3 or k_codes.dim() != 4 or v_codes.shape != k_codes.shape:
        raise ValueError("expected q [B, Hq, d] and code caches [B, Hkv, Lmax, d/2]")
    B, hq, d = q.shape
    _, hkv, L, half = k_codes.shape
    if k_codes.shape[0] != B or 2 * half != d or k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("code caches must be uint8 [B, Hkv, Lmax, d/2]")
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        if t.shape != (B, hkv, L) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [B, Hkv, Lmax]")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
        raise ValueError("kv_lens must be an int32 device tensor with one entry per sequence")
    _same_device(q, k_codes=k_codes, v_codes=v_codes, k_scales=k_scales, v_scales=v_scales)
    S = decode_q4_num_splits(B, hkv, L) if num_splits is None else int(num_splits)
    pm, pl, po = _partials(partials, B, hq, S, d, q.device)
    st = lib.attn_decode_splitk_q4(_dev(q, "q"), _dev(k_codes, "k_codes"), _dev(k_scales, "k_scales"),
                                   _dev(v_codes, "v_codes"), _dev(v_scales, "v_scales"), _dev(kv_lens, "kv_lens"), L,
                                   _dtype_code(q), B, hq, hkv, d, _scale(scale, d), int(bool(rotated)), S,
                                   _dev(pm, "part_m"), _dev(pl, "part_l"), _dev(po, "part_o"), _stream(q))
    _lib.check("attn_decode_splitk_q4", st)
    return pm, pl, po


def decode_splitk_q4_paged(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                           v_scales: torch.Tensor, block_table: torch.Tensor, kv_lens: torch.Tensor, rotated: bool,
                           num_splits: Optional[int] = None, scale: Optional[float] = None, partials=None):
    """Partial states over a paged 4-bit cache: ``k_codes, v_codes: [P, Hkv, page, d/2]`` uint8,
    ``k_scales, v_scales: [P, Hkv, page]`` fp32, ``block_table: [B, max_pages]`` int32 (device).  Same outputs
    as ``decode_splitk_q4`` over the cache the pages hold."""
    lib = _lib_handle()
    if q.dim() != 3 or k_codes.dim() != 4 or v_codes.shape != k_codes.shape or block_table.dim() != 2:
        raise ValueError("expected q [B, Hq, d], code pools [P, Hkv, page, d/2] and block_table [B, max_pages]")
    B, hq, d = q.shape
    P, hkv, page, half = k_codes.shape
    if 2 * half != d or k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("code pools must be uint8 [P, Hkv, page, d/2]")
    for name, t in (("k_scales", k_scales), ("v_scales", v_scales)):
        if t.shape != (P, hkv, page) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [P, Hkv, page]")
    if block_table.dtype != torch.int32 or block_table.shape[0] != B or block_table.device != q.device:
        raise ValueError("block_table must be an int32 device tensor [B, max_pages]")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
        raise ValueError("kv_lens must be an int32 device tensor with one entry per sequence")
    _same_device(q, k_codes=k_codes, v_codes=v_codes, k_scales=k_scales, v_scales=v_scales)
    max_pages = block_table.shape[1]
    S = decode_q4_num_splits(B, hkv, max_pages * page) if num_splits is None else int(num_splits)
    pm, pl, po = _partials(partials, B, hq, S, d, q.device)
    st = lib.attn_decode_splitk_q4_paged(_dev(q, "q"), _dev(k_codes, "k_codes"), _dev(k_scales, "k_scales"),
                                         _dev(v_codes, "v_codes"), _dev(v_scales, "v_scales"),
                                         _dev(block_table, "block_table"), max_pages, P, page,
                                         _dev(kv_lens, "kv_lens"), _dtype_code(q), B, hq, hkv, d, _scale(scale, d),
                                         int(bool(rotated)), S, _dev(pm, "part_m"), _dev(pl, "part_l"),
                                         _dev(po, "part_o"), _stream(q))
    _lib.check("attn_decode_splitk_q4_paged", st)
    return pm, pl, po


def kv_quantize_q4(x: torch.Tensor, rotated: bool, out_rows: Optional[torch.Tensor] = None,
                   codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None):
    """Encode rows ``x [..., d]`` (bf16/fp16, device) into 4-bit cache rows: returns ``(codes, scales)``,
    ``codes [..., d/2]`` uint8 and ``scales [...]`` fp32.  With ``out_rows`` (int32 device ``[rows]``) row i is
    written to row ``out_rows[i]`` of the given flat ``codes [capacity, d/2]`` / ``scales [capacity]``."""
    lib = _lib_handle()
    d = x.shape[-1]
    rows = x.numel() // d
    if (codes is None) != (scales is None):
        raise ValueError("give both codes and scales, or neither")
    if out_rows is None:
        if codes is None:
            codes = torch.empty(x.shape[:-1] + (d // 2,), dtype=torch.uint8, device=x.device)
            scales = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        _check(codes, "codes", x.shape[:-1] + (d // 2,), torch.uint8, x.device)
        _check(scales, "scales", x.shape[:-1], torch.float32, x.device)
        capacity = rows
    else:
        if codes is None:
            raise ValueError("out_rows needs the destination codes and scales")
        if out_rows.dtype != torch.int32 or out_rows.numel() != rows or out_rows.device != x.device:
            raise ValueError("out_rows must be an int32 device tensor with one entry per row")
        capacity = scales.numel()
        _check(codes, "codes", (capacity, d // 2), torch.uint8, x.device)
        _check(scales, "scales", (capacity,), torch.float32, x.device)
    st = lib.attn_kv_quantize_q4(_dev(x, "x"), rows, d, _dtype_code(x), int(bool(rotated)),
                                 None if out_rows is None else _dev(out_rows, "out_rows"), capacity,
                                 _dev(codes, "codes"), _dev(scales, "scales"), _stream(x))
    _lib.check("attn_kv_quantize_q4", st)
    return codes, scales


def merge_partials(part_m: torch.Tensor, part_l: torch.Tensor, part_o: torch.Tensor,
                   out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Merge ``[B, Hq, S]`` / ``[B, Hq, S, d]`` fp32 partials into ``[B, Hq, d]`` of ``out_dtype``."""
    lib = _lib_handle()
    if part_o.dim() != 4:
        raise ValueError("part_o must be [B, Hq, S, d]")
    B, hq, S, d = part_o.shape
    if part_m.shape != (B, hq, S) or part_l.shape != (B, hq, S):
        raise ValueError("partial shapes disagree")
    if any(t.dtype != torch.float32 for t in (part_m, part_l, part_o)):
        raise TypeError("partials must be float32")
    _same_device(part_o, part_m=part_m, part_l=part_l)
    if out is None:
        out = torch.empty((B, hq, d), dtype=out_dtype, device=part_o.device)
    elif out.dtype not in _DTYPES:
        raise ValueError(f"out must be bfloat16 or float16, got {out.dtype}")
    else:
        _check(out, "out", (B, hq, d), out.dtype, part_o.device)
    st = lib.attn_merge_partials(_dev(part_m, "part_m"), _dev(part_l, "part_l"), _dev(part_o, "part_o"), B, hq, d,
                                 S, _dev(out, "out"), _DTYPES[out.dtype], _stream(part_o))
    _lib.check("attn_merge_partials", st)
    return out


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor,
           num_splits: Optional[int] = None, scale: Optional[float] = None, partials=None) -> torch.Tensor:
    """Single-query decode: split-K partials then their merge, on the current stream."""
    pm, pl, po = decode_splitk(q, k_cache, v_cache, kv_lens, num_splits, scale, partials)
    return merge_partials(pm, pl, po, q.dtype)


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor,
                   num_splits: Optional[int] = None, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Single-query decode in one library call that allocates nothing: the split-K partial states live in
    the library's fixed per-GPU scratch array.  ``num_splits=None`` lets the library plan the split count.
    Calls that overlap on one GPU race on that array."""
    lib = _lib_handle()
    if q.dim() != 3 or k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("expected q [B, Hq, d] and caches [B, Hkv, Lmax, d]")
    B, hq, d = q.shape
    _, hkv, L, dk = k_cache.shape
    if k_cache.shape[0] != B or dk != d or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("q and caches disagree in batch, head dim or dtype")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B or kv_lens.device != q.device:
        raise ValueError("kv_lens must be an int32 device tensor with one entry per sequence")
    _same_device(q, k_cache=k_cache, v_cache=v_cache)
    out = torch.empty_like(q) if out is None else _check(out, "out", q.shape, q.dtype, q.device)
    st = lib.attn_decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                 _dev(kv_lens, "kv_lens"), L, _dtype_code(q), B, hq, hkv, d, _scale(scale, d),
                                 0 if num_splits is None else int(num_splits), _dev(out, "out"), _stream(q))
    _lib.check("attn_decode_noalloc", st)
    return out


def decode_paged(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                 kv_lens: torch.Tensor, num_splits: Optional[int] = None, scale: Optional[float] = None,
                 partials=None, window: int = 0, alibi_slopes: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Single-query decode over a paged cache: paged split-K partials then their merge."""
    pm, pl, po = decode_splitk_paged(q, k_pages, v_pages, block_table, kv_lens, num_splits, scale, partials,
                                     window, alibi_slopes)
    return merge_partials(pm, pl, po, q.dtype)


def decode_q4(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
              v_scales: torch.Tensor, kv_lens: torch.Tensor, rotated: bool, num_splits: Optional[int] = None,
              scale: Optional[float] = None, partials=None) -> torch.Tensor:
    """Single-query decode over a 4-bit cache: fused-dequant split-K partials then their merge."""
    pm, pl, po = decode_splitk_q4(q, k_codes, k_scales, v_codes, v_scales, kv_lens, rotated, num_splits, scale,
                                  partials)
    return merge_partials(pm, pl, po, q.dtype)


def decode_q4_paged(q: torch.Tensor, k_codes: torch.Tensor, k_scales: torch.Tensor, v_codes: torch.Tensor,
                    v_scales: torch.Tensor, block_table: torch.Tensor, kv_lens: torch.Tensor, rotated: bool,
                    num_splits: Optional[int] = None, scale: Optional[float] = None, partials=None) -> torch.Tensor:
    """Single-query decode over a paged 4-bit cache: fused-dequant paged split-K partials then their merge."""
    pm, pl, po = decode_splitk_q4_paged(q, k_codes, k_scales, v_codes, v_scales, block_table, kv_lens, rotated,
                                        num_splits, scale, partials)
    return merge_partials(pm, pl, po, q.dtype)
