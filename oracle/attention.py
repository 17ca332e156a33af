"""Exact softmax attention in fp64 on the CPU, written out the plain way.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

What it computes, with where each step is defined:

* ``S = Q·Kᵀ/√d``, ``P = softmax(S)`` row by row, ``O = P·V`` -- the three-line
  definition at the top of "Attention from the kernel's side: FlashAttention,
  online softmax and fused dequant", and the three steps of the "Concept"
  section of "Attention kernels".  The scale is passed in explicitly so the
  harness can hand the oracle exactly the value the GPU receives.
* Each softmax row subtracts its maximum before exponentiating ("The online
  softmax" section of the first page).  In fp64 this only matters for range,
  but it is the stated definition.
* Causal: key ``j`` is visible to query ``i`` iff ``j <= i`` ("Masking
  variants", section 5 of "Attention Computation in Practice"); the problem is
  square (as many queries as keys).
* Grouped-query attention: query head ``h`` reads KV head ``h // (Hq // Hkv)``
  ("GQA in the kernel", same section).
* Decode: one query per sequence sees keys ``0 .. kv_len-1`` of its cache and
  nothing past them ("Prefill and decode are different problems" on the first
  page; "Concept" on "Attention kernels").
* Paged decode: the same, with cache row ``j`` read from page
  ``block_table[b][j // page_size]`` at row ``j % page_size``
  ("PagedAttention's kernel difference", section 5 of "Attention Computation
  in Practice").
* A partial state ``(m, l, o)`` over a set of keys is the running maximum, the
  sum of ``exp(s_j - m)`` and the unnormalised ``sum_j exp(s_j - m) v_j``;
  two states merge by ``m = max(m_a, m_b)``, ``l = l_a e^(m_a-m) + l_b e^(m_b-m)``,
  ``o = o_a e^(m_a-m) + o_b e^(m_b-m)`` ("Maths" section of "Attention
  kernels"), where a state with ``m = -inf`` (no keys) contributes a factor 0
  (the guard in that page's "Code" section).  The output is ``o / l``.

Readings where the pages are silent (each is listed in the design doc):

* A row with no visible key (decode with ``kv_len = 0``, an all-empty merge)
  returns 0.  The pages leave softmax over no keys undefined.
* ``attention`` takes square causal problems only; ``attention_varlen``
  places a sequence's ``nq`` queries at its last ``nq`` positions
  (bottom-right alignment), which is the square rule when ``nq = nk``.

``online_softmax_tiled`` and ``split_partials`` are second implementations used
only by the oracle's own self-tests: the recurrence of "The online softmax" and
of "03 · The structure" on "Quantized kernels", and the split-K slices of
"Attention kernels".
"""

from __future__ import annotations

import math

import numpy as np

NEG_INF = float("-inf")


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """KV head read by query head ``h``: plain index arithmetic, no copy
    ("GQA in the kernel", "Attention Computation in Practice" section 5)."""
    if hkv < 1 or hq % hkv:
        raise ValueError(f"hq={hq} is not a multiple of hkv={hkv}")
    return h // (hq // hkv)


def _materialised_rows(q_rows, K, V, scale, row_index=None, window: int = 0, bias=None):
    """Softmax attention of a block of query rows over keys ``K`` / values ``V``.

    The whole block of score rows is materialised (as the textbook version on
    "Attention Computation in Practice", section 4, does one row at a time),
    offset by ``bias`` if given, masked, shifted by its row maximum,
    exponentiated, normalised by its row sum and multiplied by V.  ``row_index``
    gives each row's query position when the causal mask applies, else
    ``None``; with ``window > 0`` a row at position p also drops keys
    ``j <= p - window`` (sliding window, "Masking variants" in section 5).
    """
    S = scale * (q_rows @ K.T)
    if bias is not None:
        S = S + bias
    if row_index is not None:
        j = np.arange(K.shape[0])[None, :]
        r = np.asarray(row_index)[:, None]
        visible = j <= r
        if window > 0:
            visible = visible & (j > r - window)
        S = np.where(visible, S, -np.inf)
    if S.shape[1] == 0:
        return np.zeros((q_rows.shape[0], V.shape[1]))
    m = S.max(axis=1, keepdims=True)
    has_key = np.isfinite(m)
    E = np.exp(S - np.where(has_key, m, 0.0))  # masked scores give exp(-inf) = 0
    Z = E.sum(axis=1, keepdims=True)
    O = (E @ V) / np.where(has_key, Z, 1.0)
    return np.where(has_key, O, 0.0)


def attention(q, k, v, scale: float, causal: bool = False, row_block: int = 256):
    """Exact attention for ``q: [B, Hq, N, d]`` and ``k, v: [B, Hkv, Nk, d]``.

    Returns ``O: [B, Hq, N, d]`` in fp64.  Works per (batch, query head) over
    blocks of ``row_block`` query rows.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, N, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if causal and Nk != N:
        raise ValueError("causal attention is defined here for square problems only")
    out = np.zeros((B, Hq, N, d))
    for b in range(B):
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            for i0 in range(0, N, row_block):
                i1 = min(N, i0 + row_block)
                rows = np.arange(i0, i1) if causal else None
                out[b, h, i0:i1] = _materialised_rows(q[b, h, i0:i1], k[b, kh], v[b, kh], scale, rows)
    return out


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False, window: int = 0,
                     alibi_slopes=None):
    """Exact attention over a packed batch of sequences of different lengths.

    ``q: [total_q, Hq, d]`` and ``k, v: [total_k, Hkv, d]`` (token-major);
    sequence ``b`` owns query rows ``cu_q[b] .. cu_q[b+1]-1`` and key rows
    ``cu_k[b] .. cu_k[b+1]-1`` (the varlen "cu_seqlens" kernels of "The four
    attention kernels you actually use", section 5 of "Attention Computation
    in Practice").  Its ``nq`` queries are the last ``nq`` of its ``nk``
    positions, so query ``i`` stands at position ``i + nk - nq`` and, under
    the causal rule ``j <= position`` ("Masking variants", same section),
    sees keys ``0 .. i + nk - nq``.  A query that sees no key gives 0.
    ``window = W > 0`` (causal only) keeps keys ``p - W < j <= p`` for the
    query at position ``p``; ``alibi_slopes`` (one slope ``m_h`` per query head)
    adds ``-m_h·(p - j)`` to every score (both from "Masking variants", same
    section).  Returns ``O: [total_q, Hq, d]`` in fp64 (rows owned by no
    sequence are 0).
    """
    if window and not causal:
        raise ValueError("a sliding window is defined together with the causal mask")
    q, k, v = _f64(q), _f64(k), _f64(v)
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.zeros((total_q, Hq, d))
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        nq, nk = qe - qs, ke - ks
        if nq < 0 or nk < 0:
            raise ValueError(f"sequence {b}: offsets decrease")
        positions = np.arange(nq) + (nk - nq)
        for h in range(Hq):
            kh = kv_head_of(h, Hq, Hkv)
            bias = None
            if alibi_slopes is not None:
                bias = -float(alibi_slopes[h]) * (positions[:, None] - np.arange(nk)[None, :])
            out[qs:qe, h] = _materialised_rows(q[qs:qe, h], k[ks:ke, kh], v[ks:ke, kh], scale,
                                               positions if causal else None, window, bias)
    return out


def attention_rows(q_rows, K, V, scale: float, row_index=None):
    """Exact attention of selected query rows of one head.

    ``q_rows: [R, d]``, ``K, V: [Nk, d]``; ``row_index`` (length R) gives each
    row's position for the causal mask, or ``None`` for no mask.  Used to check
    sampled rows of outputs too large to recompute whole.
    """
    return _materialised_rows(_f64(q_rows), _f64(K), _f64(V), scale, row_index)


def softmax_probabilities(q, k, scale: float, causal: bool = False):
    """The materialised probability matrix ``P = softmax(scale·Q·Kᵀ)`` of one
    head (``q: [N, d]``, ``k: [Nk, d]``), for checks on P itself."""
    q, k = _f64(q), _f64(k)
    S = scale * (q @ k.T)
    if causal:
        i = np.arange(q.shape[0])[:, None]
        j = np.arange(k.shape[0])[None, :]
        S = np.where(j <= i, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    return E / E.sum(axis=1, keepdims=True)


def decode(q, k_cache, v_cache, kv_lens, scale: float):
    """Single-query attention over a KV cache.

    ``q: [B, Hq, d]``, ``k_cache, v_cache: [B, Hkv, Lmax, d]``, ``kv_lens: [B]``.
    Query ``(b, h)`` sees cache rows ``0 .. kv_lens[b]-1`` of KV head
    ``h // (Hq // Hkv)``; rows at or past ``kv_lens[b]`` are never read.
    Returns ``O: [B, Hq, d]`` in fp64.
    """
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = k_cache.shape[1]
    g = Hq // Hkv
    kv_head_of(0, Hq, Hkv)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(kv_lens[b])
        if not 0 <= L <= k_cache.shape[2]:
            raise ValueError(f"kv_lens[{b}]={L} outside [0, {k_cache.shape[2]}]")
        for kh in range(Hkv):
            K = _f64(k_cache[b, kh, :L])
            V = _f64(v_cache[b, kh, :L])
            out[b, kh * g:(kh + 1) * g] = _materialised_rows(q[b, kh * g:(kh + 1) * g], K, V, scale)
    return out


def gather_pages(pages, table_row, length: int, kv_head: int):
    """Logical cache rows ``0 .. length-1`` of one KV head of one sequence,
    read out of a paged pool.

    ``pages: [P, Hkv, page_size, d]``; ``table_row`` lists the sequence's
    pages in order.  Row ``j`` is row ``j % page_size`` of page
    ``table_row[j // page_size]`` ("PagedAttention's kernel difference",
    section 5 of "Attention Computation in Practice": the kernel reads block
    after block through the block table).  Entries of the table past the
    pages the length needs are not looked at.
    """
    pages = np.asarray(pages)
    ps = pages.shape[2]
    rows = np.empty((length, pages.shape[3]), dtype=pages.dtype)
    for j in range(length):
        page = int(table_row[j // ps])
        if not 0 <= page < pages.shape[0]:
            raise ValueError(f"block table names page {page}; the pool holds {pages.shape[0]}")
        rows[j] = pages[page, kv_head, j % ps]
    return rows


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, scale: float, window: int = 0, alibi_slopes=None):
    """Single-query attention over a paged KV cache.

    ``q: [B, Hq, d]``, ``k_pages, v_pages: [P, Hkv, page_size, d]``,
    ``block_table: [B, max_pages]``, ``kv_lens: [B]``.  The gather of
    ``gather_pages`` followed by the same attention as ``decode``: the pages
    change where rows live, not what is computed.  The query stands at
    position ``p = kv_len - 1``; ``window = W > 0`` keeps keys
    ``p - W < j <= p`` and ``alibi_slopes`` adds ``-m_h·(p - j)`` to the
    scores of head ``h`` ("Masking variants", same section).  Returns
    ``O: [B, Hq, d]`` in fp64.
    """
    q = _f64(q)
    B, Hq, d = q.shape
    Hkv = k_pages.shape[1]
    g = Hq // Hkv
    kv_head_of(0, Hq, Hkv)
    capacity = block_table.shape[1] * k_pages.shape[2]
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(kv_lens[b])
        if not 0 <= L <= capacity:
            raise ValueError(f"kv_lens[{b}]={L} outside [0, {capacity}]")
        for kh in range(Hkv):
            K = _f64(gather_pages(k_pages, block_table[b], L, kh))
            V = _f64(gather_pages(v_pages, block_table[b], L, kh))
            heads = np.arange(kh * g, (kh + 1) * g)
            bias = None
            if alibi_slopes is not None:
                slopes = np.asarray([float(alibi_slopes[h]) for h in heads])
                bias = -slopes[:, None] * ((L - 1) - np.arange(L))[None, :]
            out[b, heads] = _materialised_rows(q[b, heads], K, V, scale, [L - 1] * g, window, bias)
    return out


def e2m1_value(code):
    """Value of 4-bit OCP MX E2M1 codes: bit 3 sign, bits 2:1 exponent e
    (bias 1), bit 0 mantissa m; e = 0 is subnormal, 0.5·m; otherwise
    2^(e-1)·(1 + m/2)."""
    c = np.asarray(code, dtype=np.int64)
    sign = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.exp2(e - 1.0) * (1.0 + 0.5 * m))
    return np.where(sign == 1, -mag, mag)


def hadamard(d: int):
    """Normalised Sylvester-Hadamard matrix H_d / sqrt(d): H_1 = [1],
    H_2n = [[H_n, H_n], [H_n, -H_n]].  Orthogonal and symmetric."""
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != d:
        raise ValueError(f"d={d} is not a power of two")
    return h / math.sqrt(d)


def dequantize_e2m1_rows(codes, scales, rotated: bool):
    """Rows ``[..., d]`` of a 4-bit cache: byte i of a row gives element 2i
    (low nibble) and 2i+1 (high nibble), each code's value times the row's
    scale; with ``rotated`` the stored row is R·x (R = ``hadamard(d)``), so x
    is R times it."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo, hi = codes & 15, codes >> 4
    vals = np.stack([e2m1_value(lo), e2m1_value(hi)], axis=-1).reshape(codes.shape[:-1] + (2 * codes.shape[-1],))
    vals = vals * _f64(scales)[..., None]
    if rotated:
        vals = vals @ hadamard(vals.shape[-1])
    return vals


def quantize_e2m1_rows(x, rotated: bool):
    """The 4-bit cache's encoder: rows ``x [..., d]`` (values exact in fp32)
    -> ``(codes uint8 [..., d/2], scales float32 [...])``, the inverse
    direction of ``dequantize_e2m1_rows``.

    The pages give no encoder ("Why a quantised cache needs a fused kernel"
    names 4-bit codes, a per-row norm and an optional Hadamard-rotated domain
    only), so the procedure is this design's, fixed step by step in fp32 so
    that any encoder following it writes the same bytes:

    1. with ``rotated``, ``y = R·x`` as Walsh-Hadamard butterflies over the
       element index bits from bit 0 upward (the lower element ``a`` and the
       upper ``b`` become ``a + b`` and ``a - b``, each rounded to fp32), then
       one fp32 multiplication by ``1/sqrt(d)`` rounded to fp32;
    2. the row scale is ``max|y| / 6`` (fp32 division; 6 is the largest E2M1
       magnitude), or 1 for an all-zero row;
    3. each ``t = y / scale`` (fp32 division) takes the code of the E2M1
       value nearest to it -- found by measuring the distance to all eight
       magnitudes -- with a tie going to the code whose mantissa bit is clear
       (round half to even), and the sign bit set when ``t < 0``.

    A row holding NaN gets a NaN scale and code 0 everywhere (no consumer
    reads such rows: they lie past a sequence's length).
    """
    y = np.array(x, dtype=np.float32)
    d = y.shape[-1]
    if rotated:
        h = 1
        while h < d:
            blocks = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
            lower, upper = blocks[..., 0, :], blocks[..., 1, :]
            y = np.stack([lower + upper, lower - upper], axis=-2).reshape(y.shape)
            h *= 2
        y = y * np.float32(1.0 / math.sqrt(d))
    with np.errstate(invalid="ignore"):
        amax = np.abs(y).max(axis=-1)
        bad = np.isnan(amax)
        scale = np.where(amax > 0, amax / np.float32(6.0), np.float32(1.0)).astype(np.float32)
        scale[bad] = np.nan
        t = (y / np.where(bad, np.float32(1.0), scale)[..., None]).astype(np.float32)
    t[np.broadcast_to(bad[..., None], t.shape)] = 0.0
    # distances (exact in fp64: t and every magnitude are fp32 values) to the
    # magnitudes of codes 0..7, the code's low bit being its mantissa bit
    mags = np.abs(e2m1_value(np.arange(8)))
    dist = np.abs(np.abs(t.astype(np.float64))[..., None] - mags)
    best = dist.min(axis=-1, keepdims=True)
    nearest = dist == best
    even_tie = nearest & (np.arange(8) % 2 == 0)
    idx = np.where(even_tie.any(axis=-1), even_tie.argmax(axis=-1), nearest.argmax(axis=-1))
    code = idx.astype(np.uint8) | ((t < 0).astype(np.uint8) << 3)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale


def decode_q4(q, k_codes, k_scales, v_codes, v_scales, kv_lens, scale: float, rotated: bool):
    """Single-query attention over a 4-bit cache: the rows are dequantised and
    the plain ``decode`` runs on them ("Why a quantised cache needs a fused
    kernel" on "Attention from the kernel's side": fusing the dequantisation
    changes the bytes read, not the result).  Only rows below each length are
    dequantised."""
    B, Hkv, L = np.asarray(k_scales).shape
    d = 2 * np.asarray(k_codes).shape[-1]
    K = np.zeros((B, Hkv, L, d))
    V = np.zeros((B, Hkv, L, d))
    for b in range(B):
        n = int(kv_lens[b])
        K[b, :, :n] = dequantize_e2m1_rows(np.asarray(k_codes)[b, :, :n], np.asarray(k_scales)[b, :, :n], rotated)
        V[b, :, :n] = dequantize_e2m1_rows(np.asarray(v_codes)[b, :, :n], np.asarray(v_scales)[b, :, :n], rotated)
    return decode(q, K, V, kv_lens, scale)


def decode_q4_paged(q, k_codes, k_scales, v_codes, v_scales, block_table, kv_lens, scale: float, rotated: bool):
    """Single-query attention over a paged 4-bit cache.

    Pools ``k_codes, v_codes: [P, Hkv, page_size, d/2]`` uint8 and ``k_scales,
    v_scales: [P, Hkv, page_size]``; ``block_table: [B, max_pages]``.  Each
    sequence's code rows and scales are gathered through the same table as in
    ``gather_pages`` ("PagedAttention's kernel difference", section 5 of
    "Attention Computation in Practice") and ``decode_q4`` runs on the
    contiguous cache they form: paging moves rows, dequantisation fixes their
    values.  Returns ``O: [B, Hq, d]`` in fp64.
    """
    k_codes, v_codes = np.asarray(k_codes, dtype=np.uint8), np.asarray(v_codes, dtype=np.uint8)
    k_scales, v_scales = _f64(k_scales), _f64(v_scales)
    B = np.asarray(q).shape[0]
    _, Hkv, ps, half = k_codes.shape
    capacity = np.asarray(block_table).shape[1] * ps
    lens = [int(n) for n in kv_lens]
    for b, n in enumerate(lens):
        if not 0 <= n <= capacity:
            raise ValueError(f"kv_lens[{b}]={n} outside [0, {capacity}]")
    L = max([1] + lens)
    kc, vc = np.zeros((B, Hkv, L, half), np.uint8), np.zeros((B, Hkv, L, half), np.uint8)
    ks, vs = np.zeros((B, Hkv, L)), np.zeros((B, Hkv, L))
    for b, n in enumerate(lens):
        for kh in range(Hkv):
            kc[b, kh, :n] = gather_pages(k_codes, block_table[b], n, kh)
            vc[b, kh, :n] = gather_pages(v_codes, block_table[b], n, kh)
            ks[b, kh, :n] = gather_pages(k_scales[..., None], block_table[b], n, kh)[:, 0]
            vs[b, kh, :n] = gather_pages(v_scales[..., None], block_table[b], n, kh)[:, 0]
    return decode_q4(q, kc, ks, vc, vs, lens, scale, rotated)


def _merge_arrays(ma, la, oa, mb, lb, ob):
    """The two-state merge rule, elementwise over any leading shape.

    ``m = max(m_a, m_b)``; each side is weighted by ``exp(m_side - m)``, or by 0
    when that side holds no keys (``m_side = -inf``), which also keeps
    ``-inf - (-inf)`` from ever being evaluated.
    """
    m = np.maximum(ma, mb)
    m_safe = np.where(m == -np.inf, 0.0, m)
    fa = np.where(ma == -np.inf, 0.0, np.exp(np.where(ma == -np.inf, m_safe, ma) - m_safe))
    fb = np.where(mb == -np.inf, 0.0, np.exp(np.where(mb == -np.inf, m_safe, mb) - m_safe))
    l = la * fa + lb * fb
    o = oa * np.asarray(fa)[..., None] + ob * np.asarray(fb)[..., None]
    return m, l, o


def empty_partial(d: int):
    """The state of a worker that saw no keys: ``(-inf, 0, 0)``."""
    return (NEG_INF, 0.0, np.zeros(d))



def merge_pair(a, b):
    """Merge two partial states ``(m, l, o)`` into one."""
    m, l, o = _merge_arrays(_f64(a[0]), _f64(a[1]), _f64(a[2]), _f64(b[0]), _f64(b[1]), _f64(b[2]))
    return (float(m), float(l), o)


def merge_partials(m, l, o):
    """Fold partial states along their last state axis and normalise.

    ``m, l: [..., S]``, ``o: [..., S, d]`` (natural-log units: ``m`` is a
    maximum of scaled scores, ``l`` and ``o`` are taken relative to ``e^m``).
    Returns ``O = o / l`` with shape ``[..., d]``, and 0 where no partial held a
    key.
    """
    m, l, o = _f64(m), _f64(l), _f64(o)
    S = m.shape[-1]
    acc_m = np.full(m.shape[:-1], -np.inf)
    acc_l = np.zeros(m.shape[:-1])
    acc_o = np.zeros(o.shape[:-2] + (o.shape[-1],))
    for s in range(S):
        acc_m, acc_l, acc_o = _merge_arrays(acc_m, acc_l, acc_o, m[..., s], l[..., s], o[..., s, :])
    has_key = (acc_l > 0)[..., None]
    return np.where(has_key, acc_o / np.where(has_key, acc_l[..., None], 1.0), 0.0)


def split_partials(q_row, K, V, scale: float, workers: int):
    """Split-K: ``workers`` contiguous key slices, one partial state each.

    Worker ``w`` takes keys ``[w·n // W, (w+1)·n // W)``; with more workers than
    keys some slices are empty and give ``(-inf, 0, 0)``.  Each partial is the
    plain definition over its slice: ``m`` the slice's largest scaled score,
    ``l = sum exp(s_j - m)``, ``o = sum exp(s_j - m) v_j``.
    """
    q_row, K, V = _f64(q_row), _f64(K), _f64(V)
    n = K.shape[0]
    parts = []
    for w in range(workers):
        j0, j1 = (w * n) // workers, ((w + 1) * n) // workers
        if j1 <= j0:
            parts.append(empty_partial(V.shape[1]))
            continue
        s = scale * (K[j0:j1] @ q_row)
        m = float(s.max())
        e = np.exp(s - m)
        parts.append((m, float(e.sum()), e @ V[j0:j1]))
    return parts


def online_softmax_tiled(q, k, v, scale: float, causal: bool = False, tile: int = 128):
    """The online-softmax recurrence over key tiles of ``tile`` keys, one head.

    ``q: [N, d]``, ``k, v: [Nk, d]``.  Per query row the state starts at
    ``m = -inf, l = 0, o = 0``; for each tile ``m_new = max(m, max_j s_j)``,
    ``alpha = exp(m - m_new)`` (0 while ``m = -inf``),
    ``l = alpha·l + sum_j exp(s_j - m_new)``,
    ``o = alpha·o + sum_j exp(s_j - m_new)·v_j``, ``m = m_new``; finally
    ``O = o / l``.  All rows advance together; under the causal mask a row's
    keys past its own position score ``-inf`` and so change nothing.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    Nk = k.shape[0]
    if tile < 1:
        raise ValueError("tile must be >= 1")
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    o = np.zeros((N, v.shape[1]))
    rows = np.arange(N)[:, None]
    for j0 in range(0, Nk, tile):
        j1 = min(Nk, j0 + tile)
        s = scale * (q @ k[j0:j1].T)
        if causal:
            s = np.where(np.arange(j0, j1)[None, :] <= rows, s, -np.inf)
        m_new = np.maximum(m, s.max(axis=1))
        live = m_new != -np.inf
        m_new_safe = np.where(live, m_new, 0.0)
        alpha = np.where(m == -np.inf, 0.0, np.exp(np.where(m == -np.inf, m_new_safe, m) - m_new_safe))
        p = np.where(live[:, None], np.exp(s - m_new_safe[:, None]), 0.0)
        l = alpha * l + p.sum(axis=1)
        o = alpha[:, None] * o + p @ v[j0:j1]
        m = m_new
    has_key = (l > 0)[:, None]
    return np.where(has_key, o / np.where(has_key, l[:, None], 1.0), 0.0)


def fp16_exp_overflow_threshold() -> float:
    """Largest x with exp(x) finite in IEEE binary16: ln(65504) ≈ 11.09
    ("The online softmax" on the first page)."""
    return math.log(65504.0)
