"""GPU parity: the HIP kernels, called through the C ABI, against the fp64 oracle.

Tolerance (written here, applied to every output element): with
Δ = float64(GPU output) − oracle (fp64, unrounded, on the same rounded
inputs), max|Δ| <= 2e-2 and mean|Δ| <= 2e-3.  Partial states (fp32) are held
to tighter bounds derived from fp32 arithmetic, stated at each check.

Cases run at sizes the oracle finishes in seconds that still span several tiles
and a ragged tail, plus every benchmarked workload at full size in the launch
configuration the bench uses: whole outputs for the N=4096 prefill batches, the
262144-position decode (plain, paged and 4-bit), the 64-sequence ragged decode
and the append batch; the causal N=32768 prefill on a row sample over all 32 heads (computed
row by row by the oracle), and properties that hold at any size.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import q4cache
import workloads

pytestmark = pytest.mark.gpu

MAX_TOL, MEAN_TOL = 2e-2, 2e-3
DEV = "cuda"


@pytest.fixture(scope="module")
def A():
    import exact_attention_flashattention_amd as A
    A._lib.load()  # fails loudly if the HIP library is not built
    return A


def f64(t):
    return t.detach().float().cpu().double().numpy()


def assert_close(got, ref, tag):
    g = f64(got) if isinstance(got, torch.Tensor) else got
    assert np.all(np.isfinite(g)), f"{tag}: non-finite output"
    d = np.abs(g - ref)
    print(f"{tag}: max|d|={d.max():.3e} mean|d|={d.mean():.3e}", flush=True)
    assert d.max() <= MAX_TOL and d.mean() <= MEAN_TOL, tag


def announce(msg):
    print(f"[gpu case] {msg}", flush=True)


# --- prefill ---------------------------------------------------------------------------

def run_prefill_case(A, B, hq, hkv, n, d, causal, dtype, seed):
    w = workloads.Prefill(f"prefill_case_{B}_{hq}_{hkv}_{n}_{d}_{int(causal)}_{dtype}", B, hq, hkv, n, d, causal, dtype)
    announce(w.name)
    q, k, v = (t.to(DEV) for t in workloads.prefill_inputs(w, salt=seed))
    out = A.prefill_fwd(q, k, v, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.attention(f64(q), f64(k), f64(v), w.scale, causal)
    assert_close(out, ref, w.name)
    return q, k, v, out


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n", [1, 7, 64, 129, 1000])
def test_prefill_edge_lengths(A, n, d, causal, dtype):
    run_prefill_case(A, 1, 2, 1, n, d, causal, dtype, seed=n)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 4), (8, 2), (8, 1)])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_heads_and_gqa(A, hq, hkv, d, causal):
    run_prefill_case(A, 2, hq, hkv, 300, d, causal, "bf16", seed=hq * 10 + hkv)


def test_prefill_causal_1head_512_fp16_full(A):
    """The one-head causal fp16 workload (N=512, d=64), whole output."""
    w = workloads.WORKLOADS["prefill_causal_b1_h1_n512_d64_f16"]
    announce(w.name)
    q, k, v = (t.to(DEV) for t in workloads.prefill_inputs(w))
    out = A.prefill_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert_close(out, oracle.attention(f64(q), f64(k), f64(v), w.scale, True), w.name)
    # row 0 sees only key 0: its output is V row 0 exactly
    assert torch.equal(out[0, 0, 0], v[0, 0, 0])


def run_prefill_tensors(A, q, k, v, causal, scale, tag):
    out = A.prefill_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert_close(out, oracle.attention(f64(q), f64(k), f64(v), scale, causal), tag)


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "bf16"), (128, "f16")])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_large_logits(A, d, dtype, causal):
    """Q scaled by 8 (a power of two: exact after rounding): score spread ~8 in natural units, so
    exponentials without a reference would overflow fp16 and the running reference is raised often."""
    w = workloads.Prefill(f"prefill_large_logits_{d}_{dtype}", 1, 2, 1, 1000, d, causal, dtype)
    announce(w.name)
    q, k, v = workloads.prefill_inputs(w, device=DEV, salt=3)
    run_prefill_tensors(A, q * 8, k, v, causal, w.scale, w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_rising_scores_force_repeated_raises(A, d, causal):
    """Key rows of 64-key tile t scaled by 1 + 2t: each tile's row maximum passes the previous one by
    several units of log2, so the kernel raises its reference again and again along the row."""
    w = workloads.Prefill(f"prefill_rising_{d}", 1, 2, 2, 1000, d, causal, "bf16")
    announce(w.name)
    q, k, v = workloads.prefill_inputs(w, salt=5)
    growth = (1.0 + 2.0 * (torch.arange(w.n) // 64).float()).view(1, 1, -1, 1)
    k = (k.float() * growth).to(k.dtype)
    run_prefill_tensors(A, q.to(DEV), k.to(DEV), v.to(DEV), causal, w.scale, w.name)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_all_scores_far_below_zero(A, d, causal):
    """Keys = u + small noise and q = -beta·u: every score is about -200 (natural units), far below
    where exp underflows; softmax is shift-invariant, so only the noise decides the weights."""
    w = workloads.Prefill(f"prefill_negative_{d}", 1, 2, 1, 700, d, causal, "bf16")
    announce(w.name)
    _, k0, v = workloads.prefill_inputs(w, salt=7)
    u = k0[:, :, :1, :].float()                      # one key row as the common direction
    k = (u + 0.1 * k0.float()).to(torch.bfloat16)
    beta = 200.0 / float((u * u).sum()) / w.scale
    q = (-beta * u).expand(-1, w.hq, w.n, -1).contiguous().to(torch.bfloat16)
    run_prefill_tensors(A, q.to(DEV), k.to(DEV), v.to(DEV), causal, w.scale, w.name)


@pytest.mark.parametrize("name", ["prefill_b4_h32_n4096_d64_bf16", "prefill_b4_h32_n4096_d128_bf16"])
def test_prefill_n4096_whole_output(A, name):
    """The non-causal batch-4, 32-head, N=4096 workloads at full size in the benchmarked launch: every
    element of all 128 (batch, head) slices against the oracle; two launches give identical bits."""
    w = workloads.WORKLOADS[name]
    announce(w.name)
    q, k, v = workloads.prefill_inputs(w, device=DEV)
    out = A.prefill_fwd(q, k, v, causal=w.causal, scale=w.scale)
    out2 = A.prefill_fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "prefill is not deterministic"
    ref = oracle.attention(f64(q), f64(k), f64(v), w.scale, w.causal)
    assert_close(out, ref, f"{w.name} (whole output)")


@pytest.mark.parametrize("B,hq,hkv,n,d,causal,dtype", [
    (5, 20, 4, 2048, 128, False, "bf16"),   # 100 (batch, head) pairs: not a multiple of the 8 XCDs
    (5, 20, 4, 2048, 128, True, "bf16"),
    (6, 16, 16, 4096, 64, True, "f16"),
    (9, 8, 2, 4096, 64, False, "bf16"),
    (3, 24, 8, 2560, 128, True, "f16"),     # longest-first causal items of 10 different lengths
])
def test_prefill_many_items_per_compute_unit(A, B, hq, hkv, n, d, causal, dtype):
    """Square problems with several work items per compute unit, head counts that do not divide by the
    8 XCDs and GQA: the whole output equals, bit for bit, the varlen kernel's on the same rows (same
    tiles, same arithmetic, another work mapping), and a row sample of every (batch, head) slice -- the
    first and last 32 rows and 32 random ones -- matches the oracle."""
    w = workloads.Prefill(f"many_items_{B}_{hq}_{hkv}_{n}_{d}_{int(causal)}_{dtype}", B, hq, hkv, n, d, causal, dtype)
    announce(w.name)
    q, k, v = (t.to(DEV) for t in workloads.prefill_inputs(w, salt=n + d))
    sq = A.prefill_fwd(q, k, v, causal=causal, scale=w.scale)
    cu = torch.arange(0, (B + 1) * n, n, dtype=torch.int32, device=DEV)
    pq = q.transpose(1, 2).reshape(B * n, hq, d).contiguous()
    pk = k.transpose(1, 2).reshape(B * n, hkv, d).contiguous()
    pv = v.transpose(1, 2).reshape(B * n, hkv, d).contiguous()
    ref_bits = A.prefill_varlen_fwd(pq, pk, pv, cu, cu, n, n, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(sq.transpose(1, 2).reshape(B * n, hq, d), ref_bits), "square kernel != varlen kernel"
    rng = np.random.default_rng(n)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(n - 32, n), rng.integers(0, n, 32)]))
    g = hq // hkv
    got, ref = [], []
    for b in range(B):
        for h in range(hq):
            K, V = f64(k[b, h // g]), f64(v[b, h // g])
            ref.append(oracle.attention_rows(f64(q[b, h])[rows], K, V, w.scale, rows if causal else None))
            got.append(f64(sq[b, h])[rows])
    assert_close(np.concatenate(got), np.concatenate(ref), f"{w.name} (row sample of every slice)")


def c3_sample_rows(n, rng):
    """The routine row sample of the causal N=32768 workload: every row of the first and last 256-row
    blocks, every row i with i mod 128 in {0, 127} (the first and last row of each 128-row block, where
    the diagonal and the tile edges meet), and 256 random rows."""
    return np.unique(np.concatenate([np.arange(0, 256), np.arange(n - 256, n), np.arange(0, n, 128),
                                     np.arange(127, n, 128), rng.integers(0, n, 256)]))


def test_prefill_causal_gqa_32k_all_heads_row_sample(A):
    """The causal GQA N=32768 workload (32 query heads on 8 KV heads, d=128) in the benchmarked launch:
    the row sample above, for every one of the 32 query heads, against the oracle computed row by row."""
    w = workloads.WORKLOADS["prefill_causal_gqa_b1_hq32_hkv8_n32768_d128_bf16"]
    announce(w.name)
    q, k, v = workloads.prefill_inputs(w, device=DEV)
    out = A.prefill_fwd(q, k, v, causal=True, scale=w.scale)
    out2 = A.prefill_fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "prefill is not deterministic"
    assert not torch.isnan(out).any()
    rng = np.random.default_rng(7)
    g = w.hq // w.hkv
    got, ref = [], []
    for h in range(w.hq):
        rows = c3_sample_rows(w.n, rng)
        if h % g == 0:
            K, V = f64(k[0, h // g]), f64(v[0, h // g])
        qh, oh = f64(q[0, h]), f64(out[0, h])
        for r0 in range(0, len(rows), 256):
            rr = rows[r0:r0 + 256]
            ref.append(oracle.attention_rows(qh[rr], K[:rr[-1] + 1], V[:rr[-1] + 1], w.scale, rr))
            got.append(oh[rr])
        print(f"head {h}: {len(rows)} rows", flush=True)
    assert_close(np.concatenate(got), np.concatenate(ref), f"{w.name} (all heads, row sample)")


# --- varlen / append prefill ------------------------------------------------------------

def varlen_case(A, w, nq, nk, seed=0):
    announce(f"varlen {w.name} nq={nq[:8]} nk={nk[:8]}")
    q, k, v, cu_q, cu_k = w_inputs = workloads.varlen_inputs(w, device=DEV, salt=seed, nq=nq, nk=nk)
    out = A.prefill_varlen_fwd(q, k, v, cu_q.to(DEV), cu_k.to(DEV), max(nq), max(nk), causal=w.causal,
                               scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), w.scale, w.causal)
    assert_close(out, ref, f"varlen {w.name}")
    return w_inputs, out


def varlen_w(hq, hkv, d, causal, dtype):
    return workloads.Varlen(f"varlen_case_{hq}_{hkv}_{d}_{int(causal)}_{dtype}", 1, hq, hkv, d, causal, dtype,
                            (1, 1), (0, 0))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_mixed_lengths(A, causal, d, dtype):
    """Appends of 1..700 queries onto 0..1200 cached positions, an empty query
    list, a sequence with no keys, more queries than keys, tile-edge lengths."""
    nq = [1, 0, 5, 300, 17, 64, 700, 256, 40]
    nk = [1, 9, 0, 300, 1200, 65, 900, 511, 20]
    varlen_case(A, varlen_w(8, 2, d, causal, dtype), nq, nk)


@pytest.mark.parametrize("hq,hkv", [(1, 1), (8, 8), (16, 2), (12, 1)])
def test_varlen_heads_and_gqa(A, hq, hkv):
    varlen_case(A, varlen_w(hq, hkv, 128, True, "bf16"), [130, 3, 513], [1000, 4, 513])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv,n", [(4, 2, 700), (8, 2, 1100)])
def test_varlen_equal_lengths_match_square_kernel_bitwise(A, d, causal, hq, hkv, n):
    """A batch of equal square sequences through the varlen kernel gives the
    square kernel's output bit for bit (same rows per wave, same arithmetic).
    The last query tile is partial in every case; where its rows fill at most
    half the waves, one varlen workgroup serves it for several query heads
    (n=1100: 2 heads per workgroup at d=128, 4 at d=64; n=700: 2 at d=64)."""
    B = 3
    w = workloads.Prefill(f"varlen_sq_{d}_{int(causal)}_{hq}_{n}", B, hq, hkv, n, d, causal, "bf16")
    announce(w.name)
    q, k, v = (t.to(DEV) for t in workloads.prefill_inputs(w))
    sq = A.prefill_fwd(q, k, v, causal=causal, scale=w.scale)
    cu = torch.arange(0, (B + 1) * n, n, dtype=torch.int32, device=DEV)
    pq = q.transpose(1, 2).reshape(B * n, hq, d).contiguous()
    pk = k.transpose(1, 2).reshape(B * n, hkv, d).contiguous()
    pv = v.transpose(1, 2).reshape(B * n, hkv, d).contiguous()
    out = A.prefill_varlen_fwd(pq, pk, pv, cu, cu, n, n, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, sq.transpose(1, 2).reshape(B * n, hq, d))


def alibi_slopes(hq):
    """The usual geometric ALiBi slopes 2^(-8(h+1)/hq), as fp32."""
    return torch.tensor([2.0 ** (-8.0 * (h + 1) / hq) for h in range(hq)], dtype=torch.float32)


@pytest.mark.parametrize("d,dtype", [(64, "bf16"), (128, "bf16"), (128, "f16")])
@pytest.mark.parametrize("window", [1, 17, 64, 300, 5000])
def test_varlen_sliding_window(A, window, d, dtype):
    """Windows of 1 key, within a subtile, one tile, several tiles and wider
    than every sequence, on mixed append lengths (nq < nk, nq = nk, nq > nk)."""
    w = varlen_w(8, 2, d, True, dtype)
    nq, nk = [1, 300, 700, 40, 513], [9, 1200, 700, 20, 2000]
    announce(f"varlen window={window} d={d} {dtype}")
    q, k, v, cu_q, cu_k = workloads.varlen_inputs(w, device=DEV, nq=nq, nk=nk)
    out = A.prefill_varlen_fwd(q, k, v, cu_q.to(DEV), cu_k.to(DEV), max(nq), max(nk), causal=True, scale=w.scale,
                               window=window)
    torch.cuda.synchronize()
    ref = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), w.scale, True, window=window)
    assert_close(out, ref, f"varlen window={window}")


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 100)])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_alibi(A, causal, window, d):
    """ALiBi slopes 2^(-8(h+1)/H) over 16 query heads (GQA 4), alone and with a
    sliding window; non-causal ALiBi adds -m·(p - j) for keys after p too."""
    w = varlen_w(16, 4, d, causal, "bf16")
    nq, nk = [1, 300, 257, 64], [700, 1200, 257, 64]
    announce(f"varlen alibi causal={causal} window={window} d={d}")
    q, k, v, cu_q, cu_k = workloads.varlen_inputs(w, device=DEV, nq=nq, nk=nk)
    sl = alibi_slopes(16)
    out = A.prefill_varlen_fwd(q, k, v, cu_q.to(DEV), cu_k.to(DEV), max(nq), max(nk), causal=causal,
                               scale=w.scale, window=window, alibi_slopes=sl.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.attention_varlen(f64(q), f64(k), f64(v), cu_q.numpy(), cu_k.numpy(), w.scale, causal,
                                  window=window, alibi_slopes=sl.double().numpy())
    assert_close(out, ref, f"varlen alibi causal={causal} window={window}")


def test_varlen_clamps_offsets_into_the_tensors(A):
    """Offsets past the packed tensors are clamped to their ends, and a
    sequence longer than max_seqlen_k to its first max_seqlen_k keys: the
    kernel reads and writes only inside the tensors."""
    w = varlen_w(4, 2, 64, True, "bf16")
    announce("varlen clamp")
    q, k, v, cu_q, cu_k = workloads.varlen_inputs(w, device=DEV, nq=[50, 60], nk=[80, 70])
    bad_q = torch.tensor([0, 50, 999], dtype=torch.int32)  # the second sequence runs past total_q = 110
    bad_k = torch.tensor([0, 80, 4000], dtype=torch.int32)  # ... and past total_k = 150
    out = torch.zeros_like(q)
    A.prefill_varlen_fwd(q, k, v, bad_q.to(DEV), bad_k.to(DEV), 60, 80, causal=True, scale=w.scale, out=out)
    torch.cuda.synchronize()
    ref = oracle.attention_varlen(f64(q), f64(k), f64(v), [0, 50, 110], [0, 80, 150], w.scale, True)
    assert_close(out, ref, "varlen clamp")
    # max_seqlen_k = 70 keeps the first sequence's first 70 keys (its queries then stand at 20 .. 69)
    out = torch.zeros_like(q)
    A.prefill_varlen_fwd(q, k, v, cu_q.to(DEV), cu_k.to(DEV), 60, 70, causal=True, scale=w.scale, out=out)
    torch.cuda.synchronize()
    ref0 = oracle.attention_varlen(f64(q[:50]), f64(k[:70]), f64(v[:70]), [0, 50], [0, 70], w.scale, True)
    assert_close(out[:50], ref0, "varlen clamp to max_seqlen_k")


@pytest.mark.parametrize("batch", [64, 65])
def test_varlen_many_sequences(A, batch):
    """8 KV heads: 64 sequences give each XCD 64 (sequence, KV head) units,
    taken in order of key count with their work items numbered back to back;
    65 give 65, taken in index order with the longest sequence's tiles set
    aside for each.  Key counts repeat (ties in the order); some sequences
    have no queries or no keys."""
    g = np.random.default_rng(batch)
    nq = [int(x) for x in g.integers(0, 300, batch)]
    nk = [q + int(g.choice([0, 0, 64, 500])) for q in nq]
    nq[3], nk[7] = 0, 0
    varlen_case(A, varlen_w(16, 8, 128, True, "bf16"), nq, nk)


def test_varlen_speculative_verify_shapes(A):
    """A few queries (1..8 draft tokens) against long caches."""
    varlen_case(A, varlen_w(32, 8, 128, True, "bf16"), [1, 4, 8, 2], [5000, 3000, 4097, 64])


VAR = workloads.WORKLOADS["append_causal_b16_hq32_hkv8_d128_q256to2048_past0to16384_bf16"]


def test_varlen_append_full_output(A):
    """The benchmarked append batch (16 sequences, 256..2048 new queries on
    0..16384 cached positions, 32/8 heads, d=128, causal) at full size in the
    bench's launch: the whole output, sequence by sequence, against the oracle
    (≈ 25 s of fp64 on 16 host threads)."""
    announce(VAR.name)
    q, k, v, cu_q, cu_k = workloads.varlen_inputs(VAR, device=DEV)
    nq, nk = VAR.lengths()
    out = A.prefill_varlen_fwd(q, k, v, cu_q.to(DEV), cu_k.to(DEV), max(nq), max(nk), causal=True,
                               scale=VAR.scale)
    torch.cuda.synchronize()
    qf, kf, vf, got = f64(q), f64(k), f64(v), f64(out)
    cq, ck = cu_q.numpy(), cu_k.numpy()
    for b in range(VAR.batch):
        qs, qe, ks, ke = int(cq[b]), int(cq[b + 1]), int(ck[b]), int(ck[b + 1])
        announce(f"{VAR.name} sequence {b}: nq={qe - qs} nk={ke - ks}")
        ref = oracle.attention_varlen(qf[qs:qe], kf[ks:ke], vf[ks:ke], [0, qe - qs], [0, ke - ks], VAR.scale, True)
        assert_close(got[qs:qe], ref, f"{VAR.name} sequence {b}")


# --- decode ----------------------------------------------------------------------------

def decode_case(A, w, kv_lens, max_len, batch, num_splits, check_partials=True, seed=0):
    announce(f"{w.name} B={batch} L={max_len} lens={kv_lens.tolist()[:6]} S={num_splits}")
    q, kc, vc, lens = workloads.decode_inputs(w, device=DEV, salt=seed, kv_lens=kv_lens, max_kv_len=max_len,
                                              batch=batch)
    lens_d = lens.to(DEV)
    S = A.decode_num_splits(batch, w.hkv, max_len) if num_splits is None else num_splits
    pm, pl, po = A.decode_splitk(q, kc, vc, lens_d, S, w.scale)
    out = A.merge_partials(pm, pl, po, q.dtype)
    torch.cuda.synchronize()
    qf, kf, vf = f64(q), f64(kc), f64(vc)
    ref = oracle.decode(qf, kf, vf, lens.numpy(), w.scale)
    assert_close(out, ref, f"{w.name} S={S}")
    if check_partials:
        C = A.decode_chunk_len(max_len, S)
        g = w.hq // w.hkv
        pm_, pl_, po_ = f64(pm), f64(pl), f64(po)
        for b in range(batch):
            for h in range(w.hq):
                for s in range(S):
                    j0, j1 = s * C, min((s + 1) * C, int(lens[b]))
                    if j1 <= j0:
                        assert pm_[b, h, s] == -np.inf and pl_[b, h, s] == 0.0 and not po_[b, h, s].any()
                        continue
                    m, l, o = oracle.split_partials(qf[b, h], kf[b, h // g, j0:j1], vf[b, h // g, j0:j1], w.scale,
                                                    1)[0]
                    # fp32 scores and exp2 with the scale folded in: m to 1e-4·(1+|m|); l rescaled to the
                    # oracle's m to 1e-4 relative; o/l to the output tolerance
                    assert abs(pm_[b, h, s] - m) <= 1e-4 * (1 + abs(m)), (b, h, s)
                    l_adj = pl_[b, h, s] * math.exp(pm_[b, h, s] - m)
                    assert abs(l_adj - l) <= 1e-4 * l, (b, h, s)
                    assert np.max(np.abs(po_[b, h, s] / pl_[b, h, s] - o / l)) <= MAX_TOL, (b, h, s)
    return q, kc, vc, lens, out


DEC = workloads.WORKLOADS["decode_b1_hq32_hkv8_d128_len262144_bf16"]
RAG = workloads.WORKLOADS["decode_ragged_b64_hq64_hkv8_d128_len1024to32768_q8_bf16"]


@pytest.mark.parametrize("S", [1, None, 7, 200])
def test_decode_split_counts(A, S):
    """Split counts 1, the heuristic's, 7, and more splits than 64-key chunks (empty splits)."""
    decode_case(A, DEC, torch.tensor([5000], dtype=torch.int32), 5000, 1, S)


@pytest.mark.parametrize("S", [1, 4])
def test_decode_lengths_around_chunk_edges(A, S):
    """Lengths 1, 2, C-1, C, C+1, 2C+1 and Lmax-1, Lmax around the split size C."""
    Lmax = 1024
    C = A.decode_chunk_len(Lmax, S)
    Ls = sorted({1, 2, C - 1, C, min(C + 1, Lmax), min(2 * C + 1, Lmax), Lmax - 1, Lmax})
    lens = torch.tensor(Ls, dtype=torch.int32)
    decode_case(A, DEC, lens, Lmax, len(Ls), S)


def test_decode_clamps_out_of_range_lengths(A):
    """A length past the cache is read as the cache length, a negative one as 0."""
    w = DEC
    announce("decode clamp")
    q, kc, vc, _ = workloads.decode_inputs(w, device=DEV, max_kv_len=300, batch=2)
    bad = torch.tensor([305, -3], dtype=torch.int32, device=DEV)
    out = A.decode(q, kc, vc, bad, 3, w.scale)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(kc), f64(vc), [300, 0], w.scale)
    assert_close(out, ref, "decode clamp")


def test_decode_single_key_is_exact(A):
    q, kc, vc, lens, out = decode_case(A, DEC, torch.tensor([1, 1], dtype=torch.int32), 64, 2, 3)
    g = DEC.hq // DEC.hkv
    for h in range(DEC.hq):
        assert torch.equal(out[:, h], vc[:, h // g, 0]), h


def test_decode_zero_length_gives_zero(A):
    q, kc, vc, lens, out = decode_case(A, DEC, torch.tensor([0, 300], dtype=torch.int32), 512, 2, 4)
    assert not out[0].float().abs().sum().item()


@pytest.mark.parametrize("hq,hkv,d,dtype", [(4, 4, 128, "bf16"), (16, 1, 64, "bf16"), (24, 1, 128, "f16"),
                                            (32, 2, 64, "f16"), (8, 8, 64, "bf16")])
def test_decode_head_layouts(A, hq, hkv, d, dtype):
    """MHA (g=1), g=16, g=24 (two query groups per KV head), fp16 and d=64."""
    w = workloads.Decode(f"decode_case_{hq}_{hkv}_{d}_{dtype}", 3, hq, hkv, d, 700, None, 1.0, dtype)
    decode_case(A, w, torch.tensor([700, 333, 64], dtype=torch.int32), 700, 3, 5)


def test_decode_ragged_reduced(A):
    lens = torch.tensor([1024, 3000, 1500, 4096], dtype=torch.int32)
    decode_case(A, RAG, lens, 4096, 4, None)


def test_decode_long_context_full(A):
    """One sequence over a 262144-key cache, the benchmarked launch, whole output."""
    announce(DEC.name)
    q, kc, vc, lens = workloads.decode_inputs(DEC, device=DEV)
    out = A.decode(q, kc, vc, lens.to(DEV), None, DEC.scale)
    out2 = A.decode(q, kc, vc, lens.to(DEV), None, DEC.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    g = DEC.hq // DEC.hkv
    qf = f64(q)
    ref = np.zeros((1, DEC.hq, DEC.d))
    for kh in range(DEC.hkv):
        K, V = f64(kc[0, kh]), f64(vc[0, kh])
        ref[0, kh * g:(kh + 1) * g] = oracle.attention_rows(qf[0, kh * g:(kh + 1) * g], K, V, DEC.scale)
    assert_close(out, ref, DEC.name)


def test_decode_ragged_whole_output(A):
    """64 ragged sequences (lengths 1024..32768, q x8): the benchmarked launch, every sequence and head
    against the oracle (rows past each length are NaN in the cache and must never be read)."""
    announce(RAG.name)
    q, kc, vc, lens = workloads.decode_inputs(RAG, device=DEV)
    out = A.decode(q, kc, vc, lens.to(DEV), None, RAG.scale)
    out2 = A.decode(q, kc, vc, lens.to(DEV), None, RAG.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2), "decode is not deterministic"
    g = RAG.hq // RAG.hkv
    Ls = lens.numpy()
    qf = f64(q)
    ref = np.zeros((RAG.batch, RAG.hq, RAG.d))
    for b in range(RAG.batch):
        L = int(Ls[b])
        Kb, Vb = f64(kc[b, :, :L]), f64(vc[b, :, :L])
        for kh in range(RAG.hkv):
            ref[b, kh * g:(kh + 1) * g] = oracle.attention_rows(qf[b, kh * g:(kh + 1) * g], Kb[kh], Vb[kh],
                                                                RAG.scale)
        if b % 16 == 15:
            print(f"sequences 0..{b} done", flush=True)
    print(f"sum of lengths {int(Ls.sum())}", flush=True)
    assert_close(out, ref, f"{RAG.name} (whole output)")


# --- paged decode ----------------------------------------------------------------------

def paged_case(A, w, kv_lens, max_len, batch, page_size, num_splits, seed=0, spare=5):
    """Paged split-K + merge against the oracle's gather-then-attend, and the
    paged partials against the contiguous kernel's on the same logical cache
    (bit-identical when both see the same split length)."""
    announce(f"paged {w.name} B={batch} L={max_len} page={page_size} lens={kv_lens.tolist()[:6]} S={num_splits}")
    q, kc, vc, lens = workloads.decode_inputs(w, device=DEV, salt=seed, kv_lens=kv_lens, max_kv_len=max_len,
                                              batch=batch)
    kp, vp, table = workloads.paged_from_cache(kc, vc, lens, page_size, workloads.seed_for(w.name, "pages", seed),
                                               spare_pages=spare)
    lens_d, table_d = lens.to(DEV), table.to(DEV)
    capacity = table.shape[1] * page_size
    S = A.decode_num_splits(batch, w.hkv, capacity) if num_splits is None else num_splits
    pm, pl, po = A.decode_splitk_paged(q, kp, vp, table_d, lens_d, S, w.scale)
    out = A.merge_partials(pm, pl, po, q.dtype)
    cm, cl, co = A.decode_splitk(q, kc, vc, lens_d, S, w.scale)
    torch.cuda.synchronize()
    if A.decode_chunk_len(capacity, S) == A.decode_chunk_len(max_len, S):
        assert torch.equal(pm, cm) and torch.equal(pl, cl) and torch.equal(po, co), "paged != contiguous partials"
    ref = oracle.decode_paged(f64(q), f64(kp), f64(vp), table.numpy(), lens.numpy(), w.scale)
    assert_close(out, ref, f"paged {w.name} page={page_size} S={S}")
    return q, kp, vp, table, lens, out


@pytest.mark.parametrize("page_size", [16, 32, 64, 256])
@pytest.mark.parametrize("S", [None, 3])
def test_decode_paged_lengths_and_page_sizes(A, page_size, S):
    """Lengths 0, 1, 15-17 (page edges), a split edge and the full capacity."""
    lens = torch.tensor([0, 1, 15, 16, 17, 700, 1024, 1100, 2048], dtype=torch.int32)
    paged_case(A, DEC, lens, 2048, len(lens), page_size, S)


@pytest.mark.parametrize("S", [1, 2])
def test_decode_paged_split_longer_than_64_pages(A, S):
    """Splits of 1536 and 3072 keys span more than 64 pages of 16 rows, so the
    kernel reloads its per-lane copy of the block table inside a split."""
    lens = torch.tensor([3072, 2500, 1025], dtype=torch.int32)
    paged_case(A, DEC, lens, 3072, 3, 16, S)


@pytest.mark.parametrize("hq,hkv,d,dtype,page_size", [(4, 4, 128, "bf16", 16), (16, 1, 64, "bf16", 32),
                                                      (24, 1, 128, "f16", 16), (32, 2, 64, "f16", 64),
                                                      (64, 8, 128, "bf16", 128)])
def test_decode_paged_head_layouts(A, hq, hkv, d, dtype, page_size):
    w = workloads.Decode(f"decode_paged_case_{hq}_{hkv}_{d}_{dtype}", 3, hq, hkv, d, 768, None, 1.0, dtype)
    paged_case(A, w, torch.tensor([768, 333, 64], dtype=torch.int32), 768, 3, page_size, None)


def test_decode_paged_shared_pages(A):
    """Two sequences listing the same pages (a shared prefix) with equal queries
    give equal outputs; a third shares the first 4 pages and then diverges."""
    announce("paged shared pages")
    w = DEC
    hq, hkv, d, ps = w.hq, w.hkv, w.d, 16
    kp = workloads.normal((12, hkv, ps, d), "bf16", workloads.seed_for("paged_shared", "k"), DEV)
    vp = workloads.normal((12, hkv, ps, d), "bf16", workloads.seed_for("paged_shared", "v"), DEV)
    q1 = workloads.normal((1, hq, d), "bf16", workloads.seed_for("paged_shared", "q"), DEV)
    q = q1.repeat(3, 1, 1).contiguous()
    table = torch.tensor([[7, 2, 9, 4, 11, 0], [7, 2, 9, 4, 11, 0], [7, 2, 9, 4, 1, 3]], dtype=torch.int32)
    lens = torch.tensor([90, 90, 96], dtype=torch.int32)
    out = A.decode_paged(q, kp, vp, table.to(DEV), lens.to(DEV), None, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out[0], out[1])
    ref = oracle.decode_paged(f64(q), f64(kp), f64(vp), table.numpy(), lens.numpy(), w.scale)
    assert_close(out, ref, "paged shared pages")


def test_decode_paged_clamps_out_of_range_page_ids(A):
    """A page id below 0 reads page 0 and one past the pool reads the last page,
    so a bad table never reads outside the pool."""
    announce("paged clamp")
    w = DEC
    q, kc, vc, lens = workloads.decode_inputs(w, device=DEV, max_kv_len=64, batch=1)
    kp, vp, table = workloads.paged_from_cache(kc, vc, lens, 16, 11, spare_pages=0)
    P = kp.shape[0]
    bad = table.clone()
    bad[0, 1], bad[0, 3] = -7, P + 100
    out = A.decode_paged(q, kp, vp, bad.to(DEV), lens.to(DEV), None, w.scale)
    torch.cuda.synchronize()
    fixed = bad.clone()
    fixed[0, 1], fixed[0, 3] = 0, P - 1
    ref = oracle.decode_paged(f64(q), f64(kp), f64(vp), fixed.numpy(), lens.numpy(), w.scale)
    assert_close(out, ref, "paged clamp")


@pytest.mark.parametrize("window", [0, 1, 31, 32, 100, 3000])
@pytest.mark.parametrize("alibi", [False, True])
def test_decode_paged_window_and_alibi(A, window, alibi):
    """Sliding windows of 1 key, just under / at a 32-key step, across steps,
    and wider than the split size, with and without ALiBi slopes, on ragged
    lengths; the heuristic split count and 3 splits."""
    if window == 0 and not alibi:
        pytest.skip("the plain case is covered above")
    w = DEC
    lens = torch.tensor([1, 17, 700, 2048, 1500], dtype=torch.int32)
    q, kc, vc, lens = workloads.decode_inputs(w, device=DEV, kv_lens=lens, max_kv_len=2048, batch=5)
    kp, vp, table = workloads.paged_from_cache(kc, vc, lens, 16, workloads.seed_for(w.name, "pages", 3))
    sl = alibi_slopes(w.hq) if alibi else None
    for S in (None, 3):
        announce(f"paged window={window} alibi={alibi} S={S}")
        out = A.decode_paged(q, kp, vp, table.to(DEV), lens.to(DEV), S, w.scale, window=window,
                             alibi_slopes=None if sl is None else sl.to(DEV))
        torch.cuda.synchronize()
        ref = oracle.decode_paged(f64(q), f64(kp), f64(vp), table.numpy(), lens.numpy(), w.scale, window,
                                  None if sl is None else sl.double().numpy())
        assert_close(out, ref, f"paged window={window} alibi={alibi} S={S}")


def test_decode_paged_long_context_full(A):
    """The 262144-key, 32/8-head cache as 16384 scattered 16-row pages (the
    benchmarked paged launch): partials bit-identical to the contiguous kernel's,
    whole output against the oracle."""
    announce(f"paged {DEC.name}")
    q, kc, vc, lens = workloads.decode_inputs(DEC, device=DEV)
    kp, vp, table = workloads.paged_from_cache(kc, vc, lens, 16, workloads.seed_for(DEC.name, "pages"))
    lens_d, table_d = lens.to(DEV), table.to(DEV)
    S = A.decode_num_splits(1, DEC.hkv, DEC.max_kv_len)
    pm, pl, po = A.decode_splitk_paged(q, kp, vp, table_d, lens_d, S, DEC.scale)
    cm, cl, co = A.decode_splitk(q, kc, vc, lens_d, S, DEC.scale)
    out = A.merge_partials(pm, pl, po, q.dtype)
    torch.cuda.synchronize()
    assert torch.equal(pm, cm) and torch.equal(pl, cl) and torch.equal(po, co)
    del kp, vp
    g = DEC.hq // DEC.hkv
    qf = f64(q)
    ref = np.zeros((1, DEC.hq, DEC.d))
    for kh in range(DEC.hkv):
        K, V = f64(kc[0, kh]), f64(vc[0, kh])
        ref[0, kh * g:(kh + 1) * g] = oracle.attention_rows(qf[0, kh * g:(kh + 1) * g], K, V, DEC.scale)
    assert_close(out, ref, f"paged {DEC.name}")


# --- 4-bit cache, fused dequant ---------------------------------------------------------

def q4_case(A, w, kv_lens, max_len, batch, num_splits, rotated, seed=0, v_mult=None):
    announce(f"q4 {w.name} B={batch} L={max_len} lens={kv_lens.tolist()[:6]} S={num_splits} rotated={rotated}")
    q, kq, ks, vq, vs, lens = q4cache.q4_inputs(w, rotated, DEV, salt=seed, kv_lens=kv_lens, max_kv_len=max_len,
                                                batch=batch, v_mult=v_mult)
    S = A.decode_q4_num_splits(batch, w.hkv, max_len) if num_splits is None else num_splits
    out = A.decode_q4(q, kq, ks, vq, vs, lens.to(DEV), rotated, S, w.scale)
    torch.cuda.synchronize()
    ref = oracle.decode_q4(f64(q), kq.cpu().numpy(), ks.cpu().double().numpy(), vq.cpu().numpy(),
                           vs.cpu().double().numpy(), lens.numpy(), w.scale, rotated)
    if v_mult is None:
        assert_close(out, ref, f"q4 {w.name} S={S} rotated={rotated}")
    else:  # the tolerance is stated for unit-scale values: compare in units of the V scaling
        assert_close(f64(out) / v_mult, ref / v_mult, f"q4 {w.name} S={S} rotated={rotated} V x{v_mult:g}")
    return out


@pytest.mark.parametrize("rotated", [False, True])
@pytest.mark.parametrize("S", [1, None, 7])
def test_decode_q4_lengths_and_splits(A, S, rotated):
    """Lengths 1, 2, around the split size and the full cache; NaN scales and
    arbitrary codes past each length are never used."""
    lens = torch.tensor([1, 2, 63, 64, 65, 700, 1024], dtype=torch.int32)
    q4_case(A, DEC, lens, 1024, len(lens), S, rotated)


@pytest.mark.parametrize("hq,hkv,d,dtype", [(4, 4, 128, "bf16"), (16, 1, 64, "bf16"), (24, 1, 128, "f16"),
                                            (32, 2, 64, "f16"), (8, 8, 64, "bf16")])
@pytest.mark.parametrize("rotated", [False, True])
def test_decode_q4_head_layouts(A, hq, hkv, d, dtype, rotated):
    w = workloads.Decode(f"decode_q4_case_{hq}_{hkv}_{d}_{dtype}", 3, hq, hkv, d, 700, None, 1.0, dtype)
    q4_case(A, w, torch.tensor([700, 333, 64], dtype=torch.int32), 700, 3, None, rotated)


def test_decode_q4_ragged_high_scores(A):
    """The ragged workload's recipe (q x8, scores far past fp16's exp range), reduced."""
    q4_case(A, RAG, torch.tensor([1024, 3000, 1500, 4096], dtype=torch.int32), 4096, 4, None, True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("rotated", [False, True])
def test_decode_q4_fp16_large_values(A, d, rotated):
    """fp16 queries and caches whose V rows reach about 1e4 in magnitude (legal fp16 values; a row's scale is
    then ~2e3): the probabilities times the V row scales exceed the fp16 range, so the kernel must not form
    them in fp16.  Reduced lengths around the split size."""
    w = workloads.Decode(f"decode_q4_fp16_large_{d}", 3, 16, 2, d, 1024, None, 1.0, "f16")
    q4_case(A, w, torch.tensor([1024, 700, 65], dtype=torch.int32), 1024, 3, None, rotated, v_mult=8192.0)


@pytest.fixture(scope="module")
def q4_full():
    """The 262144-key cache encoded as rotated 4-bit rows by the oracle's encoder on the host, with the
    16-bit rows it came from and the oracle's output over the dequantised rows (shared by the contiguous
    and the paged full-size tests: the host encoding takes about a minute)."""
    q, kc, vc, lens = workloads.decode_inputs(DEC, device=DEV)
    kq, ks = q4cache.encode(kc, True, DEV)
    vq, vs = q4cache.encode(vc, True, DEV)
    g = DEC.hq // DEC.hkv
    qf = f64(q)
    ref = np.zeros((1, DEC.hq, DEC.d))
    for kh in range(DEC.hkv):
        K = oracle.dequantize_e2m1_rows(kq[0, kh].cpu().numpy(), ks[0, kh].cpu().double().numpy(), True)
        V = oracle.dequantize_e2m1_rows(vq[0, kh].cpu().numpy(), vs[0, kh].cpu().double().numpy(), True)
        ref[0, kh * g:(kh + 1) * g] = oracle.attention_rows(qf[0, kh * g:(kh + 1) * g], K, V, DEC.scale)
    return dict(q=q, kc=kc, vc=vc, lens=lens, kq=kq, ks=ks, vq=vq, vs=vs, ref=ref)


def test_decode_q4_long_context_full(A, q4_full):
    """The 262144-key cache encoded as rotated 4-bit rows (by the oracle's encoder on the host), the
    benchmarked launch, whole output against the oracle on the dequantised rows; the HIP encoder produces
    the same codes and scales from the same rows bit for bit."""
    announce(f"q4 {DEC.name}")
    f = q4_full
    hk, hks = A.kv_quantize_q4(f["kc"], True)
    hv, hvs = A.kv_quantize_q4(f["vc"], True)
    torch.cuda.synchronize()
    assert torch.equal(hk, f["kq"]) and torch.equal(hks, f["ks"]) and torch.equal(hv, f["vq"])
    assert torch.equal(hvs, f["vs"])
    del hk, hks, hv, hvs
    out = A.decode_q4(f["q"], f["kq"], f["ks"], f["vq"], f["vs"], f["lens"].to(DEV), True, None, DEC.scale)
    torch.cuda.synchronize()
    assert_close(out, f["ref"], f"q4 {DEC.name}")


# --- paged 4-bit cache ---------------------------------------------------------------------

def q4_paged_case(A, w, kv_lens, max_len, batch, page_size, num_splits, rotated, seed=0, spare=5):
    """Paged 4-bit split-K + merge against the oracle's gather-then-dequantise decode, and the
    paged partials against the contiguous 4-bit kernel's on the same logical cache (bit-identical
    when both see the same split length)."""
    announce(f"q4 paged {w.name} B={batch} L={max_len} page={page_size} lens={kv_lens.tolist()[:6]} "
             f"S={num_splits} rotated={rotated}")
    q, kq, ks, vq, vs, lens = q4cache.q4_inputs(w, rotated, DEV, salt=seed, kv_lens=kv_lens, max_kv_len=max_len,
                                                batch=batch)
    kp, ksp, vp, vsp, table = q4cache.paged(kq, ks, vq, vs, lens, page_size,
                                            workloads.seed_for(w.name, "q4pages", seed), spare_pages=spare)
    lens_d, table_d = lens.to(DEV), table.to(DEV)
    capacity = table.shape[1] * page_size
    S = A.decode_q4_num_splits(batch, w.hkv, capacity) if num_splits is None else num_splits
    pm, pl, po = A.decode_splitk_q4_paged(q, kp, ksp, vp, vsp, table_d, lens_d, rotated, S, w.scale)
    out = A.merge_partials(pm, pl, po, q.dtype)
    cm, cl, co = A.decode_splitk_q4(q, kq, ks, vq, vs, lens_d, rotated, S, w.scale)
    torch.cuda.synchronize()
    if A.decode_chunk_len(capacity, S) == A.decode_chunk_len(max_len, S):
        assert torch.equal(pm, cm) and torch.equal(pl, cl) and torch.equal(po, co), "paged != contiguous partials"
    ref = oracle.decode_q4_paged(f64(q), kp.cpu().numpy(), ksp.cpu().double().numpy(), vp.cpu().numpy(),
                                 vsp.cpu().double().numpy(), table.numpy(), lens.numpy(), w.scale, rotated)
    assert_close(out, ref, f"q4 paged {w.name} page={page_size} S={S} rotated={rotated}")
    return out


@pytest.mark.parametrize("rotated", [False, True])
@pytest.mark.parametrize("page_size", [16, 64, 256])
def test_decode_q4_paged_lengths_and_page_sizes(A, page_size, rotated):
    """Lengths 0, 1, 15-17 (page edges), 63-65 and the full capacity; garbage codes and NaN
    scales in spare pages and last-page tails are never used."""
    lens = torch.tensor([0, 1, 15, 16, 17, 63, 64, 65, 700, 1024], dtype=torch.int32)
    q4_paged_case(A, DEC, lens, 1024, len(lens), page_size, None, rotated)


@pytest.mark.parametrize("S", [1, 3])
def test_decode_q4_paged_split_longer_than_64_pages(A, S):
    """Splits of 1024 and 3072 keys over 16-row pages span more than 64 pages, so the kernel
    reloads its per-lane copy of the block table inside a split."""
    lens = torch.tensor([3072, 2500, 1025], dtype=torch.int32)
    q4_paged_case(A, DEC, lens, 3072, 3, 16, S, True)


@pytest.mark.parametrize("hq,hkv,d,dtype", [(16, 1, 64, "bf16"), (24, 1, 128, "f16"), (32, 2, 64, "f16")])
def test_decode_q4_paged_head_layouts(A, hq, hkv, d, dtype):
    w = workloads.Decode(f"decode_q4p_case_{hq}_{hkv}_{d}_{dtype}", 3, hq, hkv, d, 700, None, 1.0, dtype)
    q4_paged_case(A, w, torch.tensor([700, 333, 64], dtype=torch.int32), 700, 3, 32, None, True)


def test_decode_q4_paged_long_context_full(A, q4_full):
    """The same 262144-key rotated 4-bit cache in 16-row pages: whole output against the oracle on the
    dequantised rows, and the paged partials bit-identical to the contiguous kernel's."""
    announce(f"q4 paged {DEC.name}")
    f = q4_full
    q, lens = f["q"], f["lens"]
    kp, ksp, vp, vsp, table = q4cache.paged(f["kq"], f["ks"], f["vq"], f["vs"], lens, 16,
                                            workloads.seed_for(DEC.name, "q4pages", 0))
    lens_d, table_d = lens.to(DEV), table.to(DEV)
    S = A.decode_q4_num_splits(1, DEC.hkv, DEC.max_kv_len)
    pm, pl, po = A.decode_splitk_q4_paged(q, kp, ksp, vp, vsp, table_d, lens_d, True, S, DEC.scale)
    out = A.merge_partials(pm, pl, po, q.dtype)
    cm, cl, co = A.decode_splitk_q4(q, f["kq"], f["ks"], f["vq"], f["vs"], lens_d, True, S, DEC.scale)
    torch.cuda.synchronize()
    assert torch.equal(pm, cm) and torch.equal(pl, cl) and torch.equal(po, co), "paged != contiguous partials"
    assert_close(out, f["ref"], f"q4 paged {DEC.name}")


@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (64, "bf16"), (128, "f16"), (64, "f16")])
@pytest.mark.parametrize("rotated", [False, True])
def test_kv_quantize_q4_matches_the_oracle_encoder_bit_exact(A, d, dtype, rotated):
    """The HIP encoder and the oracle's encoder follow the same fixed fp32
    procedure, so codes and scales agree bit for bit; rows include an
    all-zero row (scale 1) and exact code-boundary values (every midpoint
    between E2M1 magnitudes, in a row whose scale is exactly 1)."""
    announce(f"quantize d={d} {dtype} rotated={rotated}")
    x = workloads.normal((37, 5, d), dtype, workloads.seed_for("quantize", "x", d), DEV) * 3
    x[0, 0] = 0
    x[1, 1, :8] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], dtype=x.dtype)
    x[2, 2] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * (d // 8), dtype=x.dtype)
    codes, scales = A.kv_quantize_q4(x, rotated)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.quantize_e2m1_rows(x.float().cpu().numpy(), rotated)
    assert np.array_equal(scales.cpu().numpy(), ref_s)
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert scales[0, 0].item() == 1.0 and not codes[0, 0].any()


def test_kv_quantize_q4_scatters_rows_and_skips_outside(A):
    """Appending one position per (sequence, KV head) to a [B, Hkv, L] cache:
    rows land at (b·Hkv + kh)·L + pos; a destination outside the cache is
    skipped and the rest of the cache is untouched."""
    announce("quantize scatter")
    B, hkv, L, d = 3, 2, 16, 128
    x = workloads.normal((B, hkv, d), "bf16", workloads.seed_for("quantize", "scatter"), DEV)
    pos = torch.tensor([5, 0, 15], dtype=torch.int32)
    dst = ((torch.arange(B)[:, None] * hkv + torch.arange(hkv)[None, :]) * L + pos[:, None]).to(torch.int32)
    dst[2, 1] = B * hkv * L + 7  # outside: skipped
    codes = torch.full((B * hkv * L, d // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((B * hkv * L,), -1.0, dtype=torch.float32, device=DEV)
    A.kv_quantize_q4(x, True, dst.reshape(-1).to(DEV), codes, scales)
    torch.cuda.synchronize()
    ref_c, ref_s = oracle.quantize_e2m1_rows(x.float().cpu().reshape(-1, d).numpy(), True)
    written = torch.zeros(B * hkv * L, dtype=torch.bool)
    for i, r in enumerate(dst.reshape(-1).tolist()):
        if r < B * hkv * L:
            assert np.array_equal(codes[r].cpu().numpy(), ref_c[i]) and scales[r].item() == float(ref_s[i])
            written[r] = True
    assert int(written.sum()) == B * hkv - 1
    assert (codes.cpu()[~written] == 0xAB).all() and (scales.cpu()[~written] == -1.0).all()


def test_kv_quantize_then_fused_decode(A):
    """End to end on the device: a bf16 cache encoded by the HIP encoder and read by
    the fused-dequant decode equals the oracle on the dequantised rows."""
    announce("quantize + q4 decode")
    w = DEC
    lens = torch.tensor([700, 1024, 33], dtype=torch.int32)
    q, kc, vc, lens = workloads.decode_inputs(w, device=DEV, kv_lens=lens, max_kv_len=1024, batch=3)
    kc, vc = torch.nan_to_num(kc), torch.nan_to_num(vc)  # the encoder takes finite rows
    kq, ks = A.kv_quantize_q4(kc, True)
    vq, vs = A.kv_quantize_q4(vc, True)
    out = A.decode_q4(q, kq, ks, vq, vs, lens.to(DEV), True, None, w.scale)
    torch.cuda.synchronize()
    # the oracle reads its own encoding of the same rows, which the HIP encoder's must equal
    okq, oks = q4cache.encode(kc, True, "cpu")
    ovq, ovs = q4cache.encode(vc, True, "cpu")
    assert torch.equal(kq.cpu(), okq) and torch.equal(ks.cpu(), oks)
    assert torch.equal(vq.cpu(), ovq) and torch.equal(vs.cpu(), ovs)
    ref = oracle.decode_q4(f64(q), okq.numpy(), oks.double().numpy(), ovq.numpy(), ovs.double().numpy(),
                           lens.numpy(), w.scale, True)
    assert_close(out, ref, "quantize + q4 decode")


# --- merge -----------------------------------------------------------------------------

# Few rows (15): 32-column workgroups with a pairwise tree over 32 split
# groups, and from 128 splits on 16-column workgroups over 64 groups; many
# rows (512, the threshold): whole rows, 8 or 16 groups folded at once.
@pytest.mark.parametrize("S,B,H", [(1, 3, 5), (2, 3, 5), (9, 3, 5), (127, 3, 5), (128, 3, 5), (300, 3, 5),
                                   (9, 4, 128), (130, 4, 128)])
@pytest.mark.parametrize("d,dtype", [(128, torch.bfloat16), (64, torch.float16)])
def test_merge_random_partials(A, S, B, H, d, dtype):
    announce(f"merge S={S} B={B} H={H} d={d} {dtype}")
    gen = torch.Generator().manual_seed(S * 1000 + d + B * H)
    m = torch.rand(B, H, S, generator=gen) * 40 - 5
    l = torch.rand(B, H, S, generator=gen) * 50 + 1
    o = torch.randn(B, H, S, d, generator=gen) * l[..., None]
    empty = torch.rand(B, H, S, generator=gen) < 0.3
    empty[0, 0] = True  # one row with no keys at all
    m[empty] = -math.inf
    l[empty] = 0
    o[empty] = 0
    out = A.merge_partials(m.to(DEV), l.to(DEV), o.to(DEV), dtype)
    torch.cuda.synchronize()
    ref = oracle.merge_partials(m.double().numpy(), l.double().numpy(), o.double().numpy())
    assert_close(out, ref, f"merge S={S} d={d}")
    assert not out[0, 0].float().abs().sum().item()
