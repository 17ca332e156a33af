"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This module holds shapes, random-number recipes and the accounting of
algorithmic work.  It holds none of the attention arithmetic: both the HIP
library and the fp64 oracle receive the tensors it builds, and neither imports
the other.

Recipe (every workload): entries are drawn i.i.d. N(0, 1) in fp32 from a torch
generator seeded by ``(workload, tensor)``, then rounded to the storage dtype
(bf16 or fp16) with round-to-nearest-even.  The ragged-decode workload scales
the rounded query by 8, a power of two, so the scaling is exact.  Decode caches
are ``[B, Hkv, Lmax, d]``; rows at or past a sequence's length are filled with
NaN, so that reading one would poison the output.  Small workloads are drawn
on the CPU; the large ones can be drawn directly on the GPU (a CUDA generator
gives a different, equally seeded stream), and the oracle then reads the very
tensors the GPU received.
"""

from __future__ import annotations

import dataclasses
import math
import zlib
from typing import Optional

import torch

BASE_SEED = 20240601

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "kv_lens": 4, "lens": 5, "pages": 6}


@dataclasses.dataclass(frozen=True)
class Prefill:
    """A square prefill forward: ``Q, O: [B, Hq, N, d]``, ``K, V: [B, Hkv, N, d]``."""

    name: str
    batch: int
    hq: int
    hkv: int
    n: int
    d: int
    causal: bool
    dtype: str  # "bf16" or "f16"

    @property
    def scale(self) -> float:
        return fp32_scale(self.d)

    def flops(self) -> float:
        """Algorithmic FLOPs: 4·d per visible (query, key) pair -- 2·d for the
        score dot product and 2·d for the weighted sum of V.  Masked pairs, the
        exponentials and the max/sum bookkeeping are not counted."""
        pairs = self.n * (self.n + 1) // 2 if self.causal else self.n * self.n
        return 4.0 * self.d * self.batch * self.hq * pairs

    def io_bytes(self) -> float:
        """Compulsory HBM bytes: read Q, K, V once, write O once."""
        es = 2
        return es * self.d * self.n * self.batch * (2 * self.hq + 2 * self.hkv)


@dataclasses.dataclass(frozen=True)
class Decode:
    """Single-query decode over a KV cache ``[B, Hkv, Lmax, d]``."""

    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    max_kv_len: int
    len_range: Optional[tuple]  # None: every sequence is max_kv_len long
    q_mult: float
    dtype: str

    @property
    def scale(self) -> float:
        return fp32_scale(self.d)

    def kv_bytes(self, total_len: int) -> float:
        """Algorithmic bytes: every visible K and V row read once,
        2 tensors · Hkv · d · 2 bytes per cached position."""
        return 2.0 * self.hkv * self.d * 2 * total_len


@dataclasses.dataclass(frozen=True)
class Varlen:
    """A packed batch of sequences of different lengths (append / chunked
    prefill): sequence b appends ``nq_b`` new queries to ``past_b`` cached
    positions, so it has ``nk_b = past_b + nq_b`` keys and its queries are the
    last ``nq_b`` positions.  Q, O ``[Σnq, Hq, d]``; K, V ``[Σnk, Hkv, d]``."""

    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    causal: bool
    dtype: str
    q_range: tuple     # inclusive range of nq
    past_range: tuple  # inclusive range of past

    @property
    def scale(self) -> float:
        return fp32_scale(self.d)

    def lengths(self, salt: int = 0):
        """Seeded (nq, nk) per sequence: integers uniform on the inclusive ranges."""
        gen = torch.Generator()
        gen.manual_seed(seed_for(self.name, "lens", salt) & ((1 << 63) - 1))
        nq = torch.randint(self.q_range[0], self.q_range[1] + 1, (self.batch,), generator=gen)
        past = torch.randint(self.past_range[0], self.past_range[1] + 1, (self.batch,), generator=gen)
        return [int(x) for x in nq], [int(a + b) for a, b in zip(past, nq)]

    def visible_pairs(self, nq, nk) -> int:
        """(query, key) pairs the mask leaves visible: all ``nq·nk`` without it;
        with it query i sees ``clamp(i + nk - nq + 1, 0, nk)`` keys."""
        total = 0
        for a, b in zip(nq, nk):
            if not self.causal:
                total += a * b
                continue
            i = torch.arange(a, dtype=torch.int64)
            total += int(torch.clamp(i + (b - a) + 1, 0, b).sum())
        return total

    def flops(self, nq, nk) -> float:
        """Algorithmic FLOPs: 4·d per visible (query, key) pair per query head."""
        return 4.0 * self.d * self.hq * self.visible_pairs(nq, nk)


def fp32_scale(d: int) -> float:
    """1/sqrt(d) rounded to fp32 -- the exact value the kernels receive."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32).item())


WORKLOADS = {
    w.name: w
    for w in [
        Prefill("prefill_causal_b1_h1_n512_d64_f16", 1, 1, 1, 512, 64, True, "f16"),
        Prefill("prefill_b4_h32_n4096_d64_bf16", 4, 32, 32, 4096, 64, False, "bf16"),
        Prefill("prefill_b4_h32_n4096_d128_bf16", 4, 32, 32, 4096, 128, False, "bf16"),
        Prefill("prefill_causal_gqa_b1_hq32_hkv8_n32768_d128_bf16", 1, 32, 8, 32768, 128, True, "bf16"),
        Decode("decode_b1_hq32_hkv8_d128_len262144_bf16", 1, 32, 8, 128, 262144, None, 1.0, "bf16"),
        Varlen("append_causal_b16_hq32_hkv8_d128_q256to2048_past0to16384_bf16", 16, 32, 8, 128, True, "bf16",
               (256, 2048), (0, 16384)),
        Decode("decode_ragged_b64_hq64_hkv8_d128_len1024to32768_q8_bf16", 64, 64, 8, 128, 32768,
               (1024, 32768), 8.0, "bf16"),
    ]
}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f16": torch.float16}[name]


def seed_for(workload: str, tensor: str, salt: int = 0) -> int:
    """A stable 63-bit seed from (base seed, workload name, tensor name, salt)."""
    key = f"{BASE_SEED}/{workload}/{tensor}/{salt}".encode()
    return (zlib.crc32(key) << 31) ^ (BASE_SEED * 1000003 + TENSOR_IDS.get(tensor, 0) * 7919 + salt)


def normal(shape, dtype: str, seed: int, device="cpu") -> torch.Tensor:
    """i.i.d. N(0,1) drawn in fp32 with a seeded generator, rounded (RNE) to ``dtype``."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed & ((1 << 63) - 1))
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(torch_dtype(dtype))


def prefill_inputs(w: Prefill, device="cpu", salt: int = 0, n: Optional[int] = None):
    """Q, K, V for a prefill workload (optionally with a different ``n``)."""
    n = w.n if n is None else n
    q = normal((w.batch, w.hq, n, w.d), w.dtype, seed_for(w.name, "q", salt), device)
    k = normal((w.batch, w.hkv, n, w.d), w.dtype, seed_for(w.name, "k", salt), device)
    v = normal((w.batch, w.hkv, n, w.d), w.dtype, seed_for(w.name, "v", salt), device)
    return q, k, v


def varlen_inputs(w: Varlen, device="cpu", salt: int = 0, nq=None, nk=None):
    """Packed q ``[Σnq, Hq, d]``, k and v ``[Σnk, Hkv, d]`` and the int32
    offsets ``cu_q``, ``cu_k`` (CPU) for the given or the seeded lengths."""
    if nq is None or nk is None:
        nq, nk = w.lengths(salt)
    cu_q = torch.tensor([0] + list(nq), dtype=torch.int64).cumsum(0).to(torch.int32)
    cu_k = torch.tensor([0] + list(nk), dtype=torch.int64).cumsum(0).to(torch.int32)
    q = normal((int(cu_q[-1]), w.hq, w.d), w.dtype, seed_for(w.name, "q", salt), device)
    k = normal((int(cu_k[-1]), w.hkv, w.d), w.dtype, seed_for(w.name, "k", salt), device)
    v = normal((int(cu_k[-1]), w.hkv, w.d), w.dtype, seed_for(w.name, "v", salt), device)
    return q, k, v, cu_q, cu_k


def decode_lengths(w: Decode, salt: int = 0) -> torch.Tensor:
    """Per-sequence cache lengths (int32, CPU): all ``max_kv_len``, or integers
    drawn uniformly from the inclusive range ``len_range``."""
    if w.len_range is None:
        return torch.full((w.batch,), w.max_kv_len, dtype=torch.int32)
    lo, hi = w.len_range
    gen = torch.Generator()
    gen.manual_seed(seed_for(w.name, "kv_lens", salt) & ((1 << 63) - 1))
    return torch.randint(lo, hi + 1, (w.batch,), generator=gen, dtype=torch.int64).to(torch.int32)


def decode_inputs(w: Decode, device="cpu", salt: int = 0, kv_lens: Optional[torch.Tensor] = None,
                  max_kv_len: Optional[int] = None, batch: Optional[int] = None):
    """q ``[B, Hq, d]``, NaN-padded caches ``[B, Hkv, Lmax, d]`` and lengths.

    ``batch``/``max_kv_len``/``kv_lens`` override the workload's sizes for
    reduced versions of the same recipe.
    """
    B = w.batch if batch is None else batch
    L = w.max_kv_len if max_kv_len is None else max_kv_len
    if kv_lens is None:
        kv_lens = decode_lengths(w, salt)[:B] if (batch is None and max_kv_len is None) else \
            torch.full((B,), L, dtype=torch.int32)
    kv_lens = kv_lens.to(torch.int32).cpu()
    q = normal((B, w.hq, w.d), w.dtype, seed_for(w.name, "q", salt), device)
    if w.q_mult != 1.0:
        q = q * w.q_mult  # a power of two: exact in bf16/fp16 at these magnitudes
    k = normal((B, w.hkv, L, w.d), w.dtype, seed_for(w.name, "k", salt), device)
    v = normal((B, w.hkv, L, w.d), w.dtype, seed_for(w.name, "v", salt), device)
    pad = torch.arange(L, device=device)[None, :] >= kv_lens.to(device)[:, None].long()
    if bool(pad.any()):
        k.masked_fill_(pad[:, None, :, None], float("nan"))
        v.masked_fill_(pad[:, None, :, None], float("nan"))
    return q, k, v, kv_lens


def paged_from_cache(k_cache: torch.Tensor, v_cache: torch.Tensor, kv_lens: torch.Tensor, page_size: int,
                     seed: int, spare_pages: int = 0):
    """Lay a contiguous cache ``[B, Hkv, Lmax, d]`` out as a paged pool.

    Sequence ``b`` gets ``ceil(kv_lens[b] / page_size)`` pages, taken from a
    seeded random permutation of the pool so that consecutive blocks of a
    sequence are scattered; ``spare_pages`` more pages belong to nobody.
    Returns ``(k_pages, v_pages, block_table)``: pools
    ``[P, Hkv, page_size, d]`` (NaN wherever no cache row was copied: spare
    pages and the tail of each sequence's last page) and an int32 table
    ``[B, ceil(Lmax / page_size)]`` holding -1 past each sequence's pages.
    Only rows are moved; nothing is computed.
    """
    B, hkv, L, d = k_cache.shape
    ps = page_size
    max_pages = -(-L // ps)
    lens = [int(x) for x in kv_lens.tolist()]
    need = [-(-n // ps) for n in lens]
    total = sum(need) + spare_pages
    gen = torch.Generator()
    gen.manual_seed(seed & ((1 << 63) - 1))
    perm = torch.randperm(max(total, 1), generator=gen)
    dev = k_cache.device
    pools = []
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    for cache in (k_cache, v_cache):
        pool = torch.full((max(total, 1), hkv, ps, d), float("nan"), dtype=cache.dtype, device=dev)
        pos = 0
        for b in range(B):
            n = need[b]
            if n == 0:
                continue
            ids = perm[pos:pos + n]
            table[b, :n] = ids.to(torch.int32)
            rows = cache[b, :, :min(n * ps, L)]
            if rows.shape[1] < n * ps:
                fill = torch.full((hkv, n * ps - rows.shape[1], d), float("nan"), dtype=cache.dtype, device=dev)
                rows = torch.cat([rows, fill], dim=1)
            pool[ids.to(dev)] = rows.reshape(hkv, n, ps, d).transpose(0, 1)
            pos += n
        pools.append(pool)
    return pools[0], pools[1], table


def pages_decode_kv_bytes(seq_len: int, batch: int, kv_heads: int, head_dim: int, layers: int,
                          bytes_per_value: int = 2) -> float:
    """KV bytes one decode step reads for a whole model: K and V, every layer,
    every KV head, every cached position of every sequence (the decode example
    of section 7, "Performance implications", of "Attention Computation in
    Practice")."""
    return 2.0 * layers * kv_heads * head_dim * bytes_per_value * seq_len * batch


def pages_hbm_traffic_model(n: int, d: int, sram_bytes: int, bytes_per_element: int = 2):
    """HBM elements moved for one head under the model on "Attention kernels"
    ("Maths": FlashAttention section 3.2 and Theorem 2).

    Standard attention moves ``4Nd + 4N²`` elements.  The tiled kernel, with
    ``M`` elements of SRAM, key tiles of ``B_c = ceil(M / 4d)`` and
    ``T_c = ceil(N / B_c)`` passes over the queries, moves
    ``2Nd + T_c·(3Nd + 4N)``.  Returns ``(standard_bytes, tiled_bytes,
    nxn_bytes)``; context for the bench, not a target.
    """
    M = sram_bytes // bytes_per_element
    bc = -(-M // (4 * d))
    tc = -(-n // bc)
    standard = 4 * n * d + 4 * n * n
    tiled = 2 * n * d + tc * (3 * n * d + 4 * n)
    return standard * bytes_per_element, tiled * bytes_per_element, n * n * bytes_per_element
