"""The Python binding refuses caller-supplied buffers that do not match the
call (CPU only).

The kernels write partial states at ((b·hq + h)·S + split)·d and outputs at
the shapes they are given, so a workspace or output of another shape, type or
device must be refused before anything is launched.  Every call here fails in
the binding's checks (the tensors are host or meta tensors), so no kernel runs.
"""

import pytest
import torch

import exact_attention_flashattention_amd as A

B, HQ, HKV, L, D = 2, 8, 2, 300, 128


def dec_inputs():
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    kc = torch.zeros(B, HKV, L, D, dtype=torch.bfloat16)
    lens = torch.full((B,), L, dtype=torch.int32)
    return q, kc, kc.clone(), lens


def parts(S, d=D, dtype=torch.float32, device="cpu", b=B, hq=HQ):
    return (torch.zeros(b, hq, S, dtype=dtype, device=device), torch.zeros(b, hq, S, dtype=dtype, device=device),
            torch.zeros(b, hq, S, d, dtype=dtype, device=device))


def bad_partials():
    S = 4
    good = parts(S)
    yield "part_o", (good[0], good[1], torch.zeros(B, HQ, S + 1, D))         # sized for another split count
    yield "part_m", (torch.zeros(B, HQ, S - 1), good[1], good[2])
    yield "part_l", (good[0], torch.zeros(B, HQ, S, dtype=torch.float64), good[2])
    yield "part_o", (good[0], good[1], torch.zeros(B, HQ, S, D, dtype=torch.bfloat16))
    yield "part_o", (good[0], good[1], torch.zeros(B, HQ, S, D // 2))
    yield "part_m", parts(S, device="meta")                                 # another device than q


@pytest.mark.parametrize("case", list(range(6)))
def test_decode_splitk_refuses_mismatched_partials(case):
    name, partials = list(bad_partials())[case]
    q, kc, vc, lens = dec_inputs()
    with pytest.raises(ValueError, match=name):
        A.decode_splitk(q, kc, vc, lens, 4, None, partials)


def test_decode_splitk_partials_checked_against_the_split_plan():
    """With num_splits=None the split count comes from the library's plan; a
    workspace sized for any other count is refused."""
    q, kc, vc, lens = dec_inputs()
    S = A.decode_num_splits(B, HKV, L)
    with pytest.raises(ValueError, match="part_m"):
        A.decode_splitk(q, kc, vc, lens, None, None, parts(S + 1))
    # the right size passes the workspace check and stops only at the device check
    with pytest.raises(ValueError, match="device"):
        A.decode_splitk(q, kc, vc, lens, None, None, parts(S))


def test_paged_and_q4_decode_refuse_mismatched_partials():
    q = torch.zeros(B, HQ, D, dtype=torch.bfloat16)
    pages = torch.zeros(10, HKV, 16, D, dtype=torch.bfloat16)
    table = torch.zeros(B, 5, dtype=torch.int32)
    lens = torch.full((B,), 80, dtype=torch.int32)
    with pytest.raises(ValueError, match="part_o"):
        A.decode_splitk_paged(q, pages, pages, table, lens, 3, None, (*parts(3)[:2], torch.zeros(B, HQ, 2, D)))
    codes = torch.zeros(B, HKV, L, D // 2, dtype=torch.uint8)
    scales = torch.zeros(B, HKV, L, dtype=torch.float32)
    with pytest.raises(ValueError, match="part_l"):
        A.decode_splitk_q4(q, codes, scales, codes, scales, torch.full((B,), L, dtype=torch.int32), True, 5, None,
                           (parts(5)[0], torch.zeros(B, HQ, 6), parts(5)[2]))


def test_merge_refuses_mismatched_out():
    m, l, o = parts(3)
    for out in (torch.zeros(B, HQ, D + 1, dtype=torch.bfloat16), torch.zeros(B + 1, HQ, D, dtype=torch.bfloat16),
                torch.zeros(B, HQ, D, dtype=torch.float16, device="meta")):
        with pytest.raises(ValueError, match="out"):
            A.merge_partials(m, l, o, torch.bfloat16, out=out)
    with pytest.raises(ValueError, match="out"):
        A.merge_partials(m, l, o, torch.bfloat16, out=torch.zeros(B, HQ, D, dtype=torch.float32))


def test_prefill_refuses_mismatched_out():
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    for out in (torch.zeros(1, 4, 65, 64, dtype=torch.bfloat16), torch.zeros(1, 4, 64, 64, dtype=torch.float16),
                torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16, device="meta")):
        with pytest.raises(ValueError, match="out"):
            A.prefill_fwd(q, k, k, out=out)
    qv = torch.zeros(100, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(120, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 100], dtype=torch.int32)
    with pytest.raises(ValueError, match="out"):
        A.prefill_varlen_fwd(qv, kv, kv, cu, torch.tensor([0, 120], dtype=torch.int32), 100, 120,
                             out=torch.zeros(99, 4, 64, dtype=torch.bfloat16))


def test_prefill_refuses_inputs_on_another_device():
    q = torch.zeros(1, 4, 64, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError, match="device|on"):
        A.prefill_fwd(q, k, k)


def test_kv_quantize_refuses_mismatched_destinations():
    x = torch.zeros(3, 5, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="codes"):
        A.kv_quantize_q4(x, True, None, torch.zeros(3, 5, 63, dtype=torch.uint8), torch.zeros(3, 5))
    with pytest.raises(ValueError, match="scales"):
        A.kv_quantize_q4(x, True, None, torch.zeros(3, 5, 64, dtype=torch.uint8), torch.zeros(3, 5, 1))
    with pytest.raises(ValueError, match="both"):
        A.kv_quantize_q4(x, True, None, torch.zeros(3, 5, 64, dtype=torch.uint8), None)
    rows = torch.zeros(15, dtype=torch.int32)
    with pytest.raises(ValueError, match="codes"):
        A.kv_quantize_q4(x, True, rows, torch.zeros(40, 65, dtype=torch.uint8), torch.zeros(40))
