"""The bench's work accounting, pinned to figures the pages print (CPU only)."""

import json
import math
import pathlib

import pytest

import workloads

GOLDEN = json.loads((pathlib.Path(__file__).parent / "golden" / "pages_worked_figures.json").read_text())


def test_traffic_model_reproduces_printed_widget_figures():
    g = GOLDEN["traffic_model"]
    std, tiled, nxn = workloads.pages_hbm_traffic_model(g["seq"], g["head_dim"], g["sram_bytes"],
                                                         g["bytes_per_element"])
    assert round(std / 1e6, 1) == g["printed_standard_MB"]
    assert round(tiled / 1e6, 1) == g["printed_tiled_MB"]
    assert round(nxn / 1e6, 1) == g["printed_nxn_MB"]
    assert round(std / g["bandwidth_bytes_per_s"] * 1e6, 1) == g["printed_standard_us"]
    assert round(tiled / g["bandwidth_bytes_per_s"] * 1e6, 1) == g["printed_tiled_us"]
    assert round(std / tiled, 1) == g["printed_reduction"]


def test_naive_memory_column_is_fp32_scores_and_probabilities():
    g = GOLDEN["a100_memory_table"]
    for seq, printed, step in g["rows"]:
        naive = g["batch"] * g["heads"] * 2 * seq * seq * 4  # S and P, fp32, every (batch, head)
        assert abs(naive - printed) <= step / 2 + 1e-6 * printed
    s = GOLDEN["s8192_score_buffer"]
    assert round(1 * 2 * s["seq"] ** 2 * 4 / 1e6) == s["printed_MB"]


def test_decode_kv_bytes_formula_reproduces_printed_example():
    g = GOLDEN["decode_kv_example"]
    total = workloads.pages_decode_kv_bytes(g["seq"], g["batch"], g["kv_heads"], g["head_dim"], g["layers"],
                                            g["bytes_per_value"])
    assert round(total / 1e9) == g["printed_GB"]
    assert round(total / g["bandwidth_bytes_per_s"] * 1e3) == g["printed_ms"]
    # the per-layer accounting the bench uses for its decode GB/s agrees with it
    w = workloads.Decode("x", g["batch"], g["kv_heads"] * 4, g["kv_heads"], g["head_dim"], g["seq"], None, 1.0,
                         "bf16")
    assert w.kv_bytes(g["batch"] * g["seq"]) * g["layers"] == total


def test_score_matrix_sizes():
    g = GOLDEN["score_matrix_sizes"]
    assert round(4096 ** 2 * 32 * 2 / 1e9, 1) == g["n4096_h32_fp16_GB"]
    assert 8192 ** 2 * 2 / 2 ** 20 == g["n8192_fp16_MiB"]
    assert 32768 ** 2 * 2 / 2 ** 30 == g["n32768_fp16_GiB"]


@pytest.mark.parametrize("n", [1, 2, 7, 64, 130])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_flops_count_visible_pairs(n, causal):
    w = workloads.Prefill("x", 2, 3, 1, n, 64, causal, "bf16")
    pairs = sum(1 for i in range(n) for j in range(n) if (j <= i or not causal))
    assert w.flops() == 4 * 64 * 2 * 3 * pairs


def test_workload_shapes():
    W = workloads.WORKLOADS
    assert len(W) == 7
    c3 = W["prefill_causal_gqa_b1_hq32_hkv8_n32768_d128_bf16"]
    assert math.isclose(c3.flops(), 8.796e12, rel_tol=1e-3)
    c2 = W["prefill_b4_h32_n4096_d128_bf16"]
    assert math.isclose(c2.flops(), 1.0995e12, rel_tol=1e-4)
    c4 = W["decode_b1_hq32_hkv8_d128_len262144_bf16"]
    assert c4.kv_bytes(262144) == 2 * 8 * 128 * 2 * 262144
    for w in W.values():
        assert w.hq % w.hkv == 0
        assert w.scale == pytest.approx(1 / math.sqrt(w.d), rel=1e-7)


def test_append_lengths_are_seeded_and_in_range():
    w = workloads.WORKLOADS["append_causal_b16_hq32_hkv8_d128_q256to2048_past0to16384_bf16"]
    (nq, nk), (nq2, nk2) = w.lengths(), w.lengths()
    assert nq == nq2 and nk == nk2 and len(nq) == w.batch
    assert all(256 <= a <= 2048 and 0 <= b - a <= 16384 for a, b in zip(nq, nk))


def test_ragged_lengths_are_seeded_and_in_range():
    w = workloads.WORKLOADS["decode_ragged_b64_hq64_hkv8_d128_len1024to32768_q8_bf16"]
    a, b = workloads.decode_lengths(w), workloads.decode_lengths(w)
    assert a.tolist() == b.tolist()
    assert a.min() >= 1024 and a.max() <= 32768 and len(a) == 64
