"""4-bit cache inputs for the GPU tests, encoded by the oracle's encoder.

The decode workloads' bf16/fp16 caches (from ``workloads``) are encoded on
the host with ``oracle.quantize_e2m1_rows``, one KV head at a time, and the
codes and scales are uploaded; the HIP decode and the oracle then read the
very same cache, none of it produced by the HIP path.
"""

import numpy as np
import torch

import oracle
import workloads


def encode(x: torch.Tensor, rotated: bool, device):
    """``x [..., L, d]`` (any device) -> device tensors ``codes [..., L, d/2]``
    uint8 and ``scales [..., L]`` fp32, encoded on the host."""
    lead = x.shape[:-2]
    flat = x.reshape((-1,) + tuple(x.shape[-2:]))
    codes = np.empty(flat.shape[:-1] + (x.shape[-1] // 2,), dtype=np.uint8)
    scales = np.empty(flat.shape[:-1], dtype=np.float32)
    for i in range(flat.shape[0]):
        codes[i], scales[i] = oracle.quantize_e2m1_rows(flat[i].float().cpu().numpy(), rotated)
    return (torch.from_numpy(codes).reshape(lead + codes.shape[1:]).to(device),
            torch.from_numpy(scales).reshape(lead + scales.shape[1:]).to(device))


def q4_inputs(w, rotated: bool, device, salt: int = 0, kv_lens=None, max_kv_len=None, batch=None, v_mult=None):
    """The decode workload's q and lengths with its NaN-padded caches encoded as
    4-bit rows: ``(q, k_codes, k_scales, v_codes, v_scales, kv_lens)``.
    ``v_mult`` scales the V cache before encoding (large-value cases)."""
    q, kc, vc, lens = workloads.decode_inputs(w, device, salt, kv_lens, max_kv_len, batch)
    if v_mult is not None:
        vc = (vc.float() * v_mult).to(vc.dtype)
    kq, ks = encode(kc, rotated, device)
    del kc
    vq, vs = encode(vc, rotated, device)
    return q, kq, ks, vq, vs, lens


def paged(kq, ks, vq, vs, kv_lens, page_size: int, seed: int, spare_pages: int = 0):
    """Lay a contiguous 4-bit cache (codes ``[B, Hkv, Lmax, d/2]``, scales
    ``[B, Hkv, Lmax]``) out as paged pools, as ``workloads.paged_from_cache``
    does for 16-bit caches: sequence ``b`` takes ``ceil(kv_lens[b] / page)``
    pages of a seeded random permutation, ``spare_pages`` more belong to nobody.
    Rows that no cache row was copied to (spare pages, last-page tails) hold
    code byte 0xFF and a NaN scale.  Returns ``(k_codes, k_scales, v_codes,
    v_scales, block_table)``: pools ``[P, Hkv, page, d/2]`` / ``[P, Hkv, page]``
    on the caches' device and an int32 CPU table ``[B, ceil(Lmax / page)]``
    holding -1 past each sequence's pages.  Only rows are moved."""
    B, hkv, L, half = kq.shape
    ps = page_size
    lens = [int(x) for x in kv_lens.tolist()]
    need = [-(-n // ps) for n in lens]
    total = max(1, sum(need) + spare_pages)
    gen = torch.Generator()
    gen.manual_seed(seed & ((1 << 63) - 1))
    perm = torch.randperm(total, generator=gen)
    table = torch.full((B, -(-L // ps)), -1, dtype=torch.int32)
    dev = kq.device
    pools = []
    for codes, scales in ((kq, ks), (vq, vs)):
        pc = torch.full((total, hkv, ps, half), 0xFF, dtype=torch.uint8, device=dev)
        psc = torch.full((total, hkv, ps), float("nan"), dtype=torch.float32, device=dev)
        pos = 0
        for b in range(B):
            for i in range(need[b]):
                page = int(perm[pos + i])
                table[b, i] = page
                lo, hi = i * ps, min((i + 1) * ps, lens[b])
                pc[page, :, :hi - lo] = codes[b, :, lo:hi]
                psc[page, :, :hi - lo] = scales[b, :, lo:hi]
            pos += need[b]
        pools += [pc, psc]
    return pools[0], pools[1], pools[2], pools[3], table

