"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test checks the oracle against a closed form, an invariant, a special case
that reduces to a textbook or library routine, or a figure the pages print.
They are chosen so that a plausible slip in the oracle -- a dropped term, a
wrong sign or index, a transposed operand, an off-by-one in the causal mask or
in a cache length, a wrong GQA mapping, a missing guard -- fails at least one.
"""

import json
import math
import pathlib

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = json.loads((pathlib.Path(__file__).parent / "golden" / "pages_worked_figures.json").read_text())
TOL = GOLDEN["test_contract"]["tolerance"]  # 1e-12, "Attention kernels", 'Code'


def gauss(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def one_head(q, k, v, scale, causal):
    return oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal)[0, 0]


# --- tiled recurrence vs the materialised definition ------------------------------------

@pytest.mark.parametrize("tile", [1, 2, 3, 7, 8, 64, 128, 256, 511, 512])
def test_tiled_equals_naive_at_go_example_shape(tile):
    g = GOLDEN["go_example"]
    n, d = g["seq"], g["head_dim"]
    q, k, v = gauss(1, n, d), gauss(2, n, d), gauss(3, n, d)
    scale = 1 / math.sqrt(d)
    ref = one_head(q, k, v, scale, causal=True)
    got = oracle.online_softmax_tiled(q, k, v, scale, causal=True, tile=tile)
    assert np.max(np.abs(got - ref)) <= TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tile", [1, 8, 47, 48])
def test_tiled_equals_naive_at_widget_shape(causal, tile):
    g = GOLDEN["widget_tiling"]
    nq, nk, d = g["queries"], g["keys"], g["head_dim"]
    q, k, v = gauss(4, nq, d), gauss(5, nk, d), gauss(6, nk, d)
    ref = one_head(q, k, v, 0.25, causal)
    got = oracle.online_softmax_tiled(q, k, v, 0.25, causal=causal, tile=tile)
    assert np.max(np.abs(got - ref)) <= TOL


def test_tiled_differs_from_unrescaled_variant():
    """The rescale by exp(m - m_new) matters: dropping it (keeping l and o as they
    were) gives a visibly different answer on the same data, so the agreement
    above is not vacuous."""
    n, d = 64, 16
    q, k, v = gauss(7, n, d), gauss(8, n, d), gauss(9, n, d)
    k[40] *= 6.0  # a late, large score forces a rescale
    scale = 0.5
    ref = one_head(q, k, v, scale, causal=False)
    # same recurrence with alpha forced to 1 and p taken against the *tile* max
    m = np.full(n, -np.inf); l = np.zeros(n); o = np.zeros((n, d))
    for j0 in range(0, n, 8):
        s = scale * q @ k[j0:j0 + 8].T
        m_new = np.maximum(m, s.max(1))
        p = np.exp(s - m_new[:, None])
        l = l + p.sum(1); o = o + p @ v[j0:j0 + 8]; m = m_new
    assert np.max(np.abs(o / l[:, None] - ref)) > 1e-3


# --- split-K and the merge rule --------------------------------------------------------

def fold_left(parts):
    acc = oracle.empty_partial(parts[0][2].shape[0])
    for p in parts:
        acc = oracle.merge_pair(acc, p)
    return acc


def finish(state):
    m, l, o = state
    return o / l


@pytest.mark.parametrize("workers", [1, 2, 3, 4, 7, 1000, 1500])
def test_splitk_equals_naive_1000_keys(workers):
    c = GOLDEN["test_contract"]
    n, d = c["split_keys"], 16
    q, k, v = gauss(10, d), gauss(11, n, d) * 2.0, gauss(12, n, d)
    ref = one_head(q[None], k, v, 0.25, causal=False)[0]
    parts = oracle.split_partials(q, k, v, 0.25, workers)
    assert len(parts) == workers
    if workers > n:
        assert sum(1 for p in parts if p[0] == -np.inf) == workers - n
    assert np.max(np.abs(finish(fold_left(parts)) - ref)) <= TOL
    # the array form used to check GPU partials gives the same answer
    m = np.array([p[0] for p in parts]); l = np.array([p[1] for p in parts])
    o = np.stack([p[2] for p in parts])
    assert np.max(np.abs(oracle.merge_partials(m, l, o) - ref)) <= TOL


def test_splitk_widget_4096_keys_4_workers():
    g = GOLDEN["widget_splitk"]
    d = 16
    q = gauss(13, d) * 3.0
    k, v = gauss(14, g["keys"], d), gauss(15, g["keys"], d)
    ref = one_head(q[None], k, v, 1 / math.sqrt(d), causal=False)[0]
    parts = oracle.split_partials(q, k, v, 1 / math.sqrt(d), g["workers"])
    assert np.max(np.abs(finish(fold_left(parts)) - ref)) <= TOL
    # the invariants the printed partials satisfy (their inputs are not given):
    # each slice's l lies in [1, slice length] and the merged max is the largest m_s
    slice_len = g["keys"] // g["workers"]
    for m_s, l_s, _ in parts:
        assert 1.0 <= l_s <= slice_len
    assert fold_left(parts)[0] == max(p[0] for p in parts)
    for m_s, l_s in g["printed_partials_m_l"]:
        assert 1.0 <= l_s <= slice_len
    printed_m = [m for m, _ in g["printed_partials_m_l"]]
    assert max(printed_m) == printed_m[0] == 16.81


@pytest.mark.parametrize("order", ["left", "right", "tree", "shuffled"])
def test_merge_order_does_not_matter(order):
    """'correct for any block order' (Quantized kernels, '02 · The insight')."""
    n, d = 777, 8
    q, k, v = gauss(16, d), gauss(17, n, d) * 3.0, gauss(18, n, d)
    ref = one_head(q[None], k, v, 0.3, causal=False)[0]
    parts = oracle.split_partials(q, k, v, 0.3, 13)
    if order == "left":
        st = fold_left(parts)
    elif order == "right":
        st = parts[-1]
        for p in reversed(parts[:-1]):
            st = oracle.merge_pair(p, st)
    elif order == "tree":
        level = list(parts)
        while len(level) > 1:
            nxt = [oracle.merge_pair(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
            if len(level) % 2:
                nxt.append(level[-1])
            level = nxt
        st = level[0]
    else:
        perm = np.random.default_rng(19).permutation(len(parts))
        st = fold_left([parts[i] for i in perm])
    assert np.max(np.abs(finish(st) - ref)) <= TOL


def test_merge_with_empty_is_identity_bit_exact():
    d = 16
    x = oracle.split_partials(gauss(20, d), gauss(21, 50, d), gauss(22, 50, d), 0.25, 1)[0]
    e = oracle.empty_partial(d)
    for y in (oracle.merge_pair(x, e), oracle.merge_pair(e, x)):
        assert y[0] == x[0] and y[1] == x[1]
        assert np.array_equal(y[2], x[2])
    z = oracle.merge_pair(e, e)
    assert z[0] == -np.inf and z[1] == 0.0 and not np.any(z[2])
    # all-empty array merge gives the no-key convention, 0, and no NaN
    out = oracle.merge_partials(np.full(3, -np.inf), np.zeros(3), np.zeros((3, d)))
    assert np.array_equal(out, np.zeros(d))


def test_merge_two_states_closed_form():
    """Two single-key states: the merged output must be the two-key softmax."""
    s0, s1 = 3.7, -1.2
    v0, v1 = gauss(23, 4), gauss(24, 4)
    a = (s0, 1.0, v0.copy())
    b = (s1, 1.0, v1.copy())
    sig = 1 / (1 + math.exp(-(s0 - s1)))
    expect = v1 + (v0 - v1) * sig
    assert np.max(np.abs(finish(oracle.merge_pair(a, b)) - expect)) <= 1e-14


# --- the definition itself -------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one(causal):
    n, d = 300, 32
    q, k = gauss(25, n, d) * 2, gauss(26, n, d)
    P = oracle.softmax_probabilities(q, k, 0.2, causal)
    assert np.max(np.abs(P.sum(1) - 1.0)) <= TOL
    if causal:
        assert np.all(P[np.triu_indices(n, 1)] == 0.0)
    v = gauss(27, n, d)
    assert np.max(np.abs(P @ v - one_head(q, k, v, 0.2, causal))) <= TOL


def test_single_key_returns_its_value_row_bit_exact():
    d = 64
    q, k, v = gauss(28, 1, d), gauss(29, 1, d), gauss(30, 1, d)
    assert np.array_equal(one_head(q, k, v, 0.125, causal=False), v)
    qn, kn, vn = gauss(31, 9, d), gauss(32, 9, d), gauss(33, 9, d)
    assert np.array_equal(one_head(qn, kn, vn, 0.125, causal=True)[0], vn[0])
    kc = np.full((1, 1, 5, d), np.nan); vc = np.full((1, 1, 5, d), np.nan)
    kc[0, 0, 0], vc[0, 0, 0] = kn[0], vn[0]
    out = oracle.decode(qn[:1][None], kc, vc, [1], 0.125)
    assert np.array_equal(out[0, 0], vn[0])


def test_zero_query_gives_prefix_means():
    """Q = 0 makes every visible key equally likely: row i of causal attention is
    the mean of V rows 0..i, which pins the diagonal of the mask."""
    n, d = 200, 16
    q = np.zeros((n, d)); k, v = gauss(34, n, d), gauss(35, n, d)
    expect = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(one_head(q, k, v, 0.3, causal=True) - expect)) <= TOL
    assert np.max(np.abs(one_head(q, k, v, 0.3, causal=False) - v.mean(0))) <= TOL


def test_equal_keys_give_mean_of_values():
    n, d = 123, 16
    q = gauss(36, 10, d) * 5
    k = np.repeat(gauss(37, 1, d), n, axis=0)
    v = gauss(38, n, d)
    assert np.max(np.abs(one_head(q, k, v, 0.3, causal=False) - v.mean(0))) <= TOL


def test_two_keys_closed_form():
    d = 32
    q, k, v = gauss(39, 1, d), gauss(40, 2, d), gauss(41, 2, d)
    scale = 0.17
    s0, s1 = scale * q[0] @ k[0], scale * q[0] @ k[1]
    expect = v[1] + (v[0] - v[1]) / (1 + math.exp(-(s0 - s1)))
    assert np.max(np.abs(one_head(q, k, v, scale, causal=False)[0] - expect)) <= 1e-14


def test_constant_values_are_returned_unchanged():
    n, d = 150, 8
    c = gauss(42, d)
    out = one_head(gauss(43, n, d) * 4, gauss(44, n, d), np.tile(c, (n, 1)), 0.5, causal=True)
    assert np.max(np.abs(out - c)) <= TOL


def test_permuting_keys_with_values_changes_nothing():
    n, d = 97, 16
    q, k, v = gauss(45, 20, d), gauss(46, n, d), gauss(47, n, d)
    perm = np.random.default_rng(48).permutation(n)
    a = one_head(q, k, v, 0.25, causal=False)
    b = one_head(q, k[perm], v[perm], 0.25, causal=False)
    assert np.max(np.abs(a - b)) <= TOL


def test_gqa_index_arithmetic_equals_repeat_interleave_bit_exact():
    """'GQA in the kernel': query head i reads KV head i // (h/h_kv); the copy
    made by repeat_interleave is the same computation."""
    B, hq, hkv, n, d = 2, 8, 2, 33, 16
    q, k, v = gauss(49, B, hq, n, d), gauss(50, B, hkv, n, d), gauss(51, B, hkv, n, d)
    a = oracle.attention(q, k, v, 0.25, causal=True)
    kx = np.repeat(k, hq // hkv, axis=1)
    vx = np.repeat(v, hq // hkv, axis=1)
    b = oracle.attention(q, kx, vx, 0.25, causal=True)
    assert np.array_equal(a, b)
    # and head 1 really does read KV head 0 (not head 1 mod 2)
    assert oracle.kv_head_of(1, hq, hkv) == 0 and oracle.kv_head_of(4, hq, hkv) == 1


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    B, hq, hkv, n, d = 2, 4, 2, 70, 32
    q, k, v = gauss(52, B, hq, n, d), gauss(53, B, hkv, n, d), gauss(54, B, hkv, n, d)
    scale = 1 / math.sqrt(d)
    ours = oracle.attention(q, k, v, scale, causal)
    tq = torch.from_numpy(q)
    tk = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=1)
    tv = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    assert np.max(np.abs(ours - ref.numpy())) <= TOL


def test_decode_matches_sdpa_and_ignores_rows_past_length():
    B, hq, hkv, L, d = 3, 8, 2, 40, 16
    lens = [40, 1, 17]
    q = gauss(55, B, hq, d)
    kc, vc = gauss(56, B, hkv, L, d), gauss(57, B, hkv, L, d)
    for b, n in enumerate(lens):
        kc[b, :, n:] = np.nan
        vc[b, :, n:] = np.nan
    out = oracle.decode(q, kc, vc, lens, 0.25)
    assert np.all(np.isfinite(out))
    for b, n in enumerate(lens):
        tk = torch.from_numpy(kc[b, :, :n]).repeat_interleave(hq // hkv, dim=0)
        tv = torch.from_numpy(vc[b, :, :n]).repeat_interleave(hq // hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b])[:, None], tk, tv, scale=0.25)[:, 0]
        assert np.max(np.abs(out[b] - ref.numpy())) <= TOL


def test_decode_is_the_last_row_of_causal_prefill():
    n, d = 64, 16
    q, k, v = gauss(58, n, d), gauss(59, n, d), gauss(60, n, d)
    pre = one_head(q, k, v, 0.25, causal=True)
    for L in (1, 2, 33, 64):
        dec = oracle.decode(q[L - 1][None, None], k[None, None], v[None, None], [L], 0.25)
        assert np.max(np.abs(dec[0, 0] - one_head(q[:L], k[:L], v[:L], 0.25, causal=True)[L - 1])) <= TOL
    assert np.max(np.abs(oracle.decode(q[-1][None, None], k[None, None], v[None, None], [n], 0.25)[0, 0]
                         - pre[-1])) <= TOL


def test_decode_with_no_keys_is_zero():
    out = oracle.decode(gauss(61, 1, 2, 8), np.full((1, 1, 4, 8), np.nan), np.full((1, 1, 4, 8), np.nan),
                        [0], 0.3)
    assert np.array_equal(out, np.zeros((1, 2, 8)))


# --- varlen / append ("The four attention kernels you actually use", "Masking variants",
# "Attention Computation in Practice" section 5) ---

def pack(seqs):
    """[H, n, d] arrays -> token-major [Σn, H, d] and offsets."""
    cu = np.cumsum([0] + [x.shape[1] for x in seqs])
    return np.concatenate([x.transpose(1, 0, 2) for x in seqs], axis=0), cu


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_square_sequences_equal_square_attention(causal):
    hq, hkv, d = 4, 2, 16
    ns = [1, 7, 40, 33]
    qs = [gauss(80 + i, hq, n, d) for i, n in enumerate(ns)]
    ks = [gauss(90 + i, hkv, n, d) for i, n in enumerate(ns)]
    vs = [gauss(100 + i, hkv, n, d) for i, n in enumerate(ns)]
    (q, cu), (k, _), (v, _) = pack(qs), pack(ks), pack(vs)
    out = oracle.attention_varlen(q, k, v, cu, cu, 0.3, causal)
    for i, n in enumerate(ns):
        ref = oracle.attention(qs[i][None], ks[i][None], vs[i][None], 0.3, causal)[0]
        assert np.max(np.abs(out[cu[i]:cu[i + 1]].transpose(1, 0, 2) - ref)) <= TOL


def test_varlen_append_chunks_reassemble_causal_prefill():
    """Causal prefill of 50 positions = three appended chunks [0, 12), [12, 31),
    [31, 50), each attending to every key up to its own end: the queries sit at
    the END of each chunk's keys (bottom-right), not at the start."""
    d, n = 8, 50
    q, k, v = gauss(110, 1, n, d), gauss(111, 1, n, d), gauss(112, 1, n, d)
    full = oracle.attention(q[None], k[None], v[None], 0.35, True)[0, 0]
    for c0, c1 in ((0, 12), (12, 31), (31, 50)):
        qc = q[0, c0:c1][:, None]
        kc, vc = k[0, :c1][:, None], v[0, :c1][:, None]
        out = oracle.attention_varlen(qc, kc, vc, [0, c1 - c0], [0, c1], 0.35, True)[:, 0]
        assert np.max(np.abs(out - full[c0:c1])) <= TOL
        if c0 > 0:  # top-left alignment would differ
            top_left = oracle.attention(np.pad(qc[:, 0], ((0, c0), (0, 0)))[None, None][:, :, :c1],
                                        kc[:, 0][None, None], vc[:, 0][None, None], 0.35, True)[0, 0, :c1 - c0]
            assert np.max(np.abs(top_left - full[c0:c1])) > 1e-3


def test_varlen_single_query_is_decode():
    hq, hkv, d = 6, 3, 8
    nks = [5, 1, 30]
    q = gauss(113, len(nks), hq, d)
    kc, vc = gauss(114, len(nks), hkv, 30, d), gauss(115, len(nks), hkv, 30, d)
    kp = np.concatenate([kc[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(nks)])
    vp = np.concatenate([vc[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(nks)])
    cu_k = np.cumsum([0] + nks)
    for causal in (False, True):
        out = oracle.attention_varlen(q, kp, vp, np.arange(len(nks) + 1), cu_k, 0.4, causal)
        assert np.max(np.abs(out - oracle.decode(q, kc, vc, nks, 0.4))) <= TOL


def test_varlen_more_queries_than_keys():
    """nq = 5 over nk = 3 keys, causal: the first two queries stand before
    every key and give 0; query 2 sees only key 0 and returns its V row exactly."""
    d = 4
    q, k, v = gauss(116, 5, 1, d), gauss(117, 3, 1, d), gauss(118, 3, 1, d)
    out = oracle.attention_varlen(q, k, v, [0, 5], [0, 3], 0.5, True)[:, 0]
    assert np.array_equal(out[:2], np.zeros((2, d)))
    assert np.array_equal(out[2], v[0, 0])
    full = oracle.attention(q[2:, 0][None, None], k[:, 0][None, None], v[:, 0][None, None], 0.5, True)[0, 0]
    assert np.max(np.abs(out[2:] - full)) <= TOL


def test_varlen_matches_sdpa_with_bottom_right_mask():
    """Library attention with an explicit boolean mask j <= i + nk - nq, built
    here from the definition, on a packed GQA batch with an empty sequence."""
    hq, hkv, d = 4, 2, 8
    nq, nk = [3, 0, 9, 16], [10, 4, 9, 20]
    cu_q, cu_k = np.cumsum([0] + nq), np.cumsum([0] + nk)
    q, k, v = gauss(119, cu_q[-1], hq, d), gauss(120, cu_k[-1], hkv, d), gauss(121, cu_k[-1], hkv, d)
    out = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.3, True)
    for b in range(len(nq)):
        if nq[b] == 0:
            continue
        mask = np.arange(nk[b])[None, :] <= np.arange(nq[b])[:, None] + nk[b] - nq[b]
        tq = torch.from_numpy(q[cu_q[b]:cu_q[b + 1]].transpose(1, 0, 2).copy())
        tk = torch.from_numpy(k[cu_k[b]:cu_k[b + 1]].transpose(1, 0, 2).copy()).repeat_interleave(2, dim=0)
        tv = torch.from_numpy(v[cu_k[b]:cu_k[b + 1]].transpose(1, 0, 2).copy()).repeat_interleave(2, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask),
                                                               scale=0.3)
        assert np.max(np.abs(out[cu_q[b]:cu_q[b + 1]] - ref.numpy().transpose(1, 0, 2))) <= TOL


def test_sliding_window_with_zero_queries_is_a_moving_average():
    """Q = 0 makes every visible key equally likely, so the output at position
    p is the mean of V over (p - W, p] (computed here with running sums)."""
    n, d, W = 40, 3, 7
    v = gauss(122, n, 1, d)
    k = gauss(123, n, 1, d)
    out = oracle.attention_varlen(np.zeros((n, 1, d)), k, v, [0, n], [0, n], 0.5, True, window=W)[:, 0]
    csum = np.concatenate([np.zeros((1, d)), np.cumsum(v[:, 0], axis=0)])
    for p_ in range(n):
        lo = max(0, p_ - W + 1)
        assert np.max(np.abs(out[p_] - (csum[p_ + 1] - csum[lo]) / (p_ + 1 - lo))) <= TOL


def test_window_covering_every_key_changes_nothing_bit_exact():
    q, k, v = gauss(124, 9, 2, 8), gauss(125, 30, 1, 8), gauss(126, 30, 1, 8)
    a = oracle.attention_varlen(q, k, v, [0, 9], [0, 30], 0.3, True)
    assert np.array_equal(oracle.attention_varlen(q, k, v, [0, 9], [0, 30], 0.3, True, window=30), a)
    assert np.array_equal(oracle.attention_varlen(q, k, v, [0, 9], [0, 30], 0.3, True, window=10 ** 6), a)
    assert not np.array_equal(oracle.attention_varlen(q, k, v, [0, 9], [0, 30], 0.3, True, window=29), a)
    with pytest.raises(ValueError):
        oracle.attention_varlen(q, k, v, [0, 9], [0, 30], 0.3, False, window=4)


def test_alibi_with_zero_queries_is_a_geometric_average():
    """Q = 0 and slope m: key j at distance p - j gets weight r^(p-j), r = e^-m;
    the weighted mean is summed here term by term."""
    n, d = 25, 2
    m = np.array([0.3, 1.1])
    v = gauss(127, n, 1, d)
    out = oracle.attention_varlen(np.zeros((n, 2, d)), gauss(128, n, 1, d), v, [0, n], [0, n], 0.25, True,
                                  alibi_slopes=m)
    for h in range(2):
        r = math.exp(-m[h])
        for p_ in range(n):
            num = sum(r ** (p_ - j) * v[j, 0] for j in range(p_ + 1))
            den = sum(r ** (p_ - j) for j in range(p_ + 1))
            assert np.max(np.abs(out[p_, h] - num / den)) <= TOL


def test_alibi_slope_zero_is_plain_attention_bit_exact_and_matches_sdpa():
    hq, d, nq, nk = 4, 8, 6, 20
    q, k, v = gauss(129, nq, hq, d), gauss(130, nk, 2, d), gauss(131, nk, 2, d)
    plain = oracle.attention_varlen(q, k, v, [0, nq], [0, nk], 0.4, True)
    assert np.array_equal(oracle.attention_varlen(q, k, v, [0, nq], [0, nk], 0.4, True,
                                                  alibi_slopes=np.zeros(hq)), plain)
    slopes = np.array([0.5, 0.25, 0.125, 0.0625])
    got = oracle.attention_varlen(q, k, v, [0, nq], [0, nk], 0.4, True, window=9, alibi_slopes=slopes)
    for h in range(hq):
        bias = np.full((nq, nk), -np.inf)
        for i in range(nq):
            p_ = i + nk - nq
            for j in range(nk):
                if p_ - 9 < j <= p_:
                    bias[i, j] = -slopes[h] * (p_ - j)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[:, h][None]), torch.from_numpy(k[:, h // 2][None]),
            torch.from_numpy(v[:, h // 2][None]), attn_mask=torch.from_numpy(bias), scale=0.4)[0]
        assert np.max(np.abs(got[:, h] - ref.numpy())) <= TOL


def test_varlen_visible_pair_count():
    w = workloads.Varlen("t", 3, 1, 1, 64, True, "bf16", (1, 1), (0, 0))
    # nq=nk=4: 1+2+3+4; nq=2 of nk=5: 4+5; nq=5 of nk=3: 0+0+1+2+3
    assert w.visible_pairs([4, 2, 5], [4, 5, 3]) == 10 + 9 + 6
    w2 = dataclasses_replace(w, causal=False)
    assert w2.visible_pairs([4, 2, 5], [4, 5, 3]) == 16 + 10 + 15


def dataclasses_replace(w, **kw):
    import dataclasses
    return dataclasses.replace(w, **kw)


# --- paged decode ("PagedAttention's kernel difference", "Attention Computation in Practice" section 5) ---

def test_gather_pages_reads_the_listed_blocks_in_order():
    """Every pool element encodes (page, head, row); with table [2, 0, 3] and
    page size 4, logical rows 0-3 come from page 2, rows 4-7 from page 0 and
    rows 8-9 from page 3, in row order -- written out by hand below."""
    P, H, ps, d = 4, 2, 4, 3
    pool = np.zeros((P, H, ps, d))
    for p_ in range(P):
        for h in range(H):
            for r in range(ps):
                pool[p_, h, r] = 100 * p_ + 10 * h + r
    got = oracle.gather_pages(pool, [2, 0, 3, 1], 10, 1)
    want = [210, 211, 212, 213, 10, 11, 12, 13, 310, 311]
    assert np.array_equal(got[:, 0], np.array(want, dtype=float))
    assert np.array_equal(got, np.repeat(got[:, :1], d, axis=1))
    assert oracle.gather_pages(pool, [2, 0, 3, 1], 0, 0).shape == (0, d)
    with pytest.raises(ValueError):
        oracle.gather_pages(pool, [2, 7], 8, 0)


def contiguous_as_identity_pages(kc, ps):
    """Pool in which sequence b's block i is page b·nblk + i (no permutation)."""
    B, H, L, d = kc.shape
    nblk = L // ps
    pool = kc.reshape(B, H, nblk, ps, d).transpose(0, 2, 1, 3, 4).reshape(B * nblk, H, ps, d)
    table = np.arange(B * nblk).reshape(B, nblk)
    return pool, table


@pytest.mark.parametrize("ps", [1, 4, 16])
def test_paged_decode_with_identity_table_is_contiguous_decode_bit_exact(ps):
    B, hq, hkv, L, d = 3, 8, 2, 48, 16
    lens = [48, 1, 17]
    q = gauss(70, B, hq, d)
    kc, vc = gauss(71, B, hkv, L, d), gauss(72, B, hkv, L, d)
    kp, table = contiguous_as_identity_pages(kc, ps)
    vp, _ = contiguous_as_identity_pages(vc, ps)
    assert np.array_equal(oracle.decode_paged(q, kp, vp, table, lens, 0.25), oracle.decode(q, kc, vc, lens, 0.25))


def test_paged_decode_scattered_pages_match_sdpa_and_skip_unused_rows():
    """Pages in a seeded random order, NaN in spare pages and in each
    sequence's last-page tail: the output equals library attention over the
    first kv_len rows."""
    B, hq, hkv, L, d, ps = 3, 8, 2, 64, 16, 16
    lens = torch.tensor([64, 1, 33], dtype=torch.int32)
    q = gauss(73, B, hq, d)
    kc, vc = gauss(74, B, hkv, L, d), gauss(75, B, hkv, L, d)
    for b, n in enumerate(lens.tolist()):
        kc[b, :, n:] = np.nan
        vc[b, :, n:] = np.nan
    kp, vp, table = workloads.paged_from_cache(torch.from_numpy(kc), torch.from_numpy(vc), lens, ps, seed=5,
                                               spare_pages=3)
    kp, vp, table = kp.numpy(), vp.numpy(), table.numpy()
    assert sorted(table[table >= 0].tolist()) != list(range(int((table >= 0).sum())))  # really scattered
    out = oracle.decode_paged(q, kp, vp, table, lens.numpy(), 0.25)
    assert np.all(np.isfinite(out))
    for b, n in enumerate(lens.tolist()):
        tk = torch.from_numpy(kc[b, :, :n]).repeat_interleave(hq // hkv, dim=0)
        tv = torch.from_numpy(vc[b, :, :n]).repeat_interleave(hq // hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b])[:, None], tk, tv, scale=0.25)[:, 0]
        assert np.max(np.abs(out[b] - ref.numpy())) <= TOL


def test_paged_decode_shared_pages_give_equal_outputs():
    """Two sequences whose tables list the same pages (a shared prefix) and
    whose queries are equal produce equal outputs; a different length does not."""
    hq, hkv, d, ps = 4, 1, 8, 4
    pool_k, pool_v = gauss(76, 6, hkv, ps, d), gauss(77, 6, hkv, ps, d)
    q1 = gauss(78, 1, hq, d)
    q = np.concatenate([q1, q1, q1])
    table = np.array([[5, 1, 3], [5, 1, 3], [5, 1, 0]])
    out = oracle.decode_paged(q, pool_k, pool_v, table, [10, 10, 12], 0.5)
    assert np.array_equal(out[0], out[1])
    assert not np.array_equal(out[0], out[2])


@pytest.mark.parametrize("window,alibi", [(0, False), (5, False), (0, True), (12, True), (1, True)])
def test_paged_decode_masks_equal_last_row_of_varlen(window, alibi):
    """Decode with a window / ALiBi = the varlen oracle with one query per
    sequence (standing at position kv_len - 1), which takes its masks from a
    separately written path; slopes 2^-(h+1)."""
    B, hq, hkv, L, d, ps = 3, 4, 2, 48, 8, 16
    lens = [48, 1, 30]
    q = gauss(132, B, hq, d)
    kc, vc = gauss(133, B, hkv, L, d), gauss(134, B, hkv, L, d)
    kp, table = contiguous_as_identity_pages(kc, ps)
    vp, _ = contiguous_as_identity_pages(vc, ps)
    slopes = 2.0 ** -(np.arange(hq) + 1.0) if alibi else None
    got = oracle.decode_paged(q, kp, vp, table, lens, 0.3, window, slopes)
    kpk = np.concatenate([kc[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)])
    vpk = np.concatenate([vc[b, :, :n].transpose(1, 0, 2) for b, n in enumerate(lens)])
    ref = oracle.attention_varlen(q, kpk, vpk, np.arange(B + 1), np.cumsum([0] + lens), 0.3, True, window, slopes)
    assert np.max(np.abs(got - ref)) <= TOL
    if window:
        assert np.max(np.abs(got - oracle.decode_paged(q, kp, vp, table, lens, 0.3, 0, slopes))) > 1e-3


# --- 4-bit cache (E2M1 codes, row scales, optional Hadamard rotation) ---

def test_e2m1_code_values():
    """All 16 codes, written out from the format's bit fields by hand."""
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    got = oracle.e2m1_value(np.arange(16))
    assert np.array_equal(got, np.array(want, dtype=float))
    assert np.signbit(got[8]) and not np.signbit(got[0])


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 64, 128])
def test_hadamard_is_scipy_hadamard_normalised_and_its_own_inverse(d):
    import scipy.linalg
    R = oracle.hadamard(d)
    assert np.array_equal(R * math.sqrt(d), scipy.linalg.hadamard(d).astype(float))
    assert np.max(np.abs(R @ R - np.eye(d))) <= 1e-14 and np.array_equal(R, R.T)


def test_dequantize_nibble_order_and_scale():
    """Bytes 0x21, 0xF1, 0xA5 hold (low, high) nibbles (1, 2), (1, 15), (5, 10):
    values (0.5, 1), (0.5, -6), (3, -1), times the row scale 0.75."""
    got = oracle.dequantize_e2m1_rows(np.array([[0x21, 0xF1, 0xA5]], dtype=np.uint8), np.array([0.75]), False)
    assert np.array_equal(got, 0.75 * np.array([[0.5, 1, 0.5, -6, 3, -1]]))
    rot = oracle.dequantize_e2m1_rows(np.array([[0x21, 0xF1]], dtype=np.uint8), np.array([2.0]), True)
    plain = 2.0 * np.array([0.5, 1, 0.5, -6])
    H = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]) / 2.0
    assert np.max(np.abs(rot[0] - H @ plain)) <= 1e-15


@pytest.mark.parametrize("rotated", [False, True])
def test_encoder_decoder_round_trip_within_half_a_step(rotated):
    """The oracle's encoder and decoder agree: each element lands on the
    nearest E2M1 magnitude, so the error in the stored domain is at most half
    the gap around it times the scale (the largest half gap is 1, between 4 and
    6); the rotation preserves the error's norm; each row's largest element is
    stored as ±6 exactly."""
    x = torch.randn(64, 128, generator=torch.Generator().manual_seed(3), dtype=torch.float32).numpy()
    codes, scales = oracle.quantize_e2m1_rows(x, rotated)
    assert codes.dtype == np.uint8 and codes.shape == (64, 64) and scales.dtype == np.float32
    back = oracle.dequantize_e2m1_rows(codes, scales, rotated)
    xs = x.astype(np.float64) @ (oracle.hadamard(128) if rotated else np.eye(128))
    bs = back @ (oracle.hadamard(128) if rotated else np.eye(128))
    t = np.abs(xs) / scales.astype(np.float64)[:, None]
    half_gap = np.select([t <= 2, t <= 4], [0.25, 0.5], 1.0)
    assert np.all(np.abs(bs - xs) <= half_gap * scales.astype(np.float64)[:, None] * (1 + 1e-6))
    assert np.allclose(np.linalg.norm(back - x.astype(np.float64), axis=1), np.linalg.norm(bs - xs, axis=1))
    assert np.all(np.abs(t).max(axis=1) <= 6 * (1 + 1e-6))
    assert np.allclose(np.abs(bs).max(axis=1), 6.0 * scales.astype(np.float64), rtol=1e-12, atol=0)


def test_encoder_ties_go_to_the_even_code():
    """A row whose largest magnitude is 6 has scale 1, so its values are
    encoded as they are.  Every midpoint between neighbouring E2M1 magnitudes
    goes to the code whose mantissa bit is clear: 0.25 -> 0 (code 0),
    0.75 -> 1 (2), 1.25 -> 1 (2), 1.75 -> 2 (4), 2.5 -> 2 (4), 3.5 -> 4 (6),
    5 -> 4 (6), 6 -> 6 (7); bytes pair (low, high) nibbles.  Just off each
    midpoint the nearer value wins, and negative values set bit 3."""
    ties = np.array([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]], dtype=np.float32)
    codes, scales = oracle.quantize_e2m1_rows(ties, False)
    assert scales.tolist() == [1.0]
    assert codes.tolist() == [[0x20, 0x42, 0x64, 0x76]]
    codes, _ = oracle.quantize_e2m1_rows(-ties, False)
    assert codes.tolist() == [[0xA8, 0xCA, 0xEC, 0xFE]]
    near = np.array([[0.26, 0.74, 1.26, 1.74, 2.51, 3.49, 5.01, -6.0]], dtype=np.float32)
    codes, _ = oracle.quantize_e2m1_rows(near, False)
    assert codes.tolist() == [[0x11, 0x33, 0x55, 0xF7]]


def test_encoder_scale_zero_row_and_rotation_by_hand():
    """Scale = max|y| / 6 in fp32; an all-zero row has scale 1 and code 0
    everywhere.  Rotated, x = (1, 2, 3, 4) becomes H_4·x / 2 = (5, -1, -2, 0)
    (butterflies over bit 0: (3, -1, 7, -1); bit 1: (10, -2, -4, 0); times
    1/2), scale 5/6, t = (6, -1.2, -2.4, 0) -> codes 7, 8|2, 8|4, 0."""
    codes, scales = oracle.quantize_e2m1_rows(np.zeros((2, 16), dtype=np.float32), True)
    assert scales.tolist() == [1.0, 1.0] and not codes.any()
    x = np.array([[1.0, 2.0, 3.0, 4.0]], dtype=np.float32)
    codes, scales = oracle.quantize_e2m1_rows(x, True)
    assert scales[0] == np.float32(5.0) / np.float32(6.0)
    assert codes.tolist() == [[0xA7, 0x0C]]
    H4 = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]]) / 2.0
    assert np.array_equal(H4 @ x[0].astype(np.float64), [5.0, -1.0, -2.0, 0.0])
    codes, scales = oracle.quantize_e2m1_rows(np.array([[3.0, -12.0, 1.0, 0.0]], dtype=np.float32), False)
    assert scales.tolist() == [2.0] and codes.tolist() == [[0xF3, 0x01]]  # t = (1.5, -6, 0.5, 0)
    nan_row = np.array([[1.0, np.nan, 2.0, 3.0]], dtype=np.float32)
    codes, scales = oracle.quantize_e2m1_rows(nan_row, False)
    assert np.isnan(scales[0]) and not codes.any()


def test_decode_q4_is_decode_on_dequantised_rows_and_single_key_exact():
    B, hq, hkv, L, d = 2, 4, 2, 40, 16
    rng = np.random.default_rng(140)
    kc = rng.integers(0, 256, (B, hkv, L, d // 2), dtype=np.uint8)
    vc = rng.integers(0, 256, (B, hkv, L, d // 2), dtype=np.uint8)
    ks, vs = rng.uniform(0.1, 1, (B, hkv, L)), rng.uniform(0.1, 1, (B, hkv, L))
    q = gauss(141, B, hq, d)
    for rotated in (False, True):
        got = oracle.decode_q4(q, kc, ks, vc, vs, [40, 1], 0.25, rotated)
        K = oracle.dequantize_e2m1_rows(kc, ks, rotated)
        V = oracle.dequantize_e2m1_rows(vc, vs, rotated)
        assert np.max(np.abs(got - oracle.decode(q, K, V, [40, 1], 0.25))) <= TOL
        # one key: its V row (exactly when unrotated; the rotated row through a different matmul shape)
        single = np.repeat(V[1, :, 0], hq // hkv, axis=0)
        assert np.array_equal(got[1], single) if not rotated else np.max(np.abs(got[1] - single)) <= TOL


def q4_pages(codes, scales, lens, ps, seed, spare=0):
    """Lay a contiguous 4-bit cache (codes [B, H, L, d/2], scales [B, H, L]) out
    as shuffled pages: each sequence takes ceil(len / ps) pages of a seeded
    permutation; spare pages and last-page tails hold code 0xFF (-6 at both
    nibbles) and a NaN scale, which no consumer may read."""
    B, H, L, half = codes.shape
    need = [-(-int(n) // ps) for n in lens]
    total = max(1, sum(need) + spare)
    perm = np.random.default_rng(seed).permutation(total)
    pc = np.full((total, H, ps, half), 0xFF, np.uint8)
    pscale = np.full((total, H, ps), np.nan)
    table = np.full((B, -(-L // ps)), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        for i in range(n):
            page = perm[pos + i]
            table[b, i] = page
            rows = slice(i * ps, min((i + 1) * ps, int(lens[b])))
            cnt = rows.stop - rows.start
            pc[page, :, :cnt] = codes[b, :, rows]
            pscale[page, :, :cnt] = scales[b, :, rows]
        pos += n
    return pc, pscale, table


@pytest.mark.parametrize("ps", [1, 4, 16])
def test_decode_q4_paged_is_decode_q4_of_the_gathered_cache(ps):
    """Pages in a seeded order (garbage in spare pages and tails): bit-identical
    to the contiguous 4-bit decode, and within TOL of library attention over the
    dequantised rows of each sequence."""
    B, hq, hkv, L, d = 3, 4, 2, 40, 16
    lens = [40, 1, 17]
    rng = np.random.default_rng(150 + ps)
    kc = rng.integers(0, 256, (B, hkv, L, d // 2), dtype=np.uint8)
    vc = rng.integers(0, 256, (B, hkv, L, d // 2), dtype=np.uint8)
    ks, vs = rng.uniform(0.1, 1, (B, hkv, L)), rng.uniform(0.1, 1, (B, hkv, L))
    q = gauss(151, B, hq, d)
    kp, ksp, table = q4_pages(kc, ks, lens, ps, seed=ps, spare=3)
    vp, vsp, table_v = q4_pages(vc, vs, lens, ps, seed=ps, spare=3)
    assert np.array_equal(table, table_v)
    if ps > 1:
        assert sorted(table[table >= 0].tolist()) != list(range(int((table >= 0).sum())))  # really scattered
    for rotated in (False, True):
        got = oracle.decode_q4_paged(q, kp, ksp, vp, vsp, table, lens, 0.25, rotated)
        assert np.array_equal(got, oracle.decode_q4(q, kc, ks, vc, vs, lens, 0.25, rotated))
        for b, n in enumerate(lens):
            K = torch.from_numpy(oracle.dequantize_e2m1_rows(kc[b, :, :n], ks[b, :, :n], rotated))
            V = torch.from_numpy(oracle.dequantize_e2m1_rows(vc[b, :, :n], vs[b, :, :n], rotated))
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b])[:, None], K.repeat_interleave(hq // hkv, dim=0),
                V.repeat_interleave(hq // hkv, dim=0), scale=0.25)[:, 0]
            assert np.max(np.abs(got[b] - ref.numpy())) <= TOL
    with pytest.raises(ValueError):
        oracle.decode_q4_paged(q, kp, ksp, vp, vsp, table, [table.shape[1] * ps + 1, 1, 17], 0.25, False)


def test_attention_rows_matches_full_output():
    B, hq, n, d = 1, 2, 130, 32
    q, k, v = gauss(62, B, hq, n, d), gauss(63, B, hq, n, d), gauss(64, B, hq, n, d)
    full = oracle.attention(q, k, v, 0.2, causal=True)
    rows = np.array([0, 1, 63, 64, 129])
    part = oracle.attention_rows(q[0, 1, rows], k[0, 1], v[0, 1], 0.2, rows)
    assert np.max(np.abs(part - full[0, 1, rows])) <= TOL


# --- range: why max subtraction is required ---------------------------------------------

def test_fp16_exp_overflow_threshold():
    g = GOLDEN["fp16_exp_overflow"]
    x = oracle.fp16_exp_overflow_threshold()
    assert round(x, 1) == g["printed_threshold"]
    assert math.isclose(math.exp(x), g["largest_fp16"], rel_tol=1e-12)
    assert float(torch.tensor(math.exp(x + 0.01)).half()) == math.inf
    assert float(torch.tensor(math.exp(x - 0.01)).half()) < math.inf


def test_ragged_decode_recipe_exceeds_fp16_exp_range():
    """The ×8 query of the ragged-decode workload drives scaled scores past
    ln(65504); the oracle still returns finite outputs because it subtracts the max."""
    w = workloads.WORKLOADS["decode_ragged_b64_hq64_hkv8_d128_len1024to32768_q8_bf16"]
    q, k, v, lens = workloads.decode_inputs(w, batch=2, max_kv_len=1024)
    qf, kf = q.double().numpy(), k.double().numpy()
    g = w.hq // w.hkv
    smax = max(float((w.scale * kf[b, h // g] @ qf[b, h]).max()) for b in range(2) for h in range(w.hq))
    assert smax > oracle.fp16_exp_overflow_threshold()
    out = oracle.decode(qf, kf, v.double().numpy(), lens.numpy(), w.scale)
    assert np.all(np.isfinite(out))
