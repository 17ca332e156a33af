"""attn_decode_noalloc -- the decode entry point that allocates nothing -- against
the entry points it stands for (attn_decode_splitk + attn_merge_partials with a
caller-owned workspace) and against the oracle.

The partial states live in the library's fixed per-GPU scratch array, which
keeps whatever the previous call left; consecutive calls, the second one
smaller, must each give exactly what the workspace path gives on the same
inputs and split count.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"
DEC = workloads.WORKLOADS["decode_b1_hq32_hkv8_d128_len262144_bf16"]
RAG = workloads.WORKLOADS["decode_ragged_b64_hq64_hkv8_d128_len1024to32768_q8_bf16"]


@pytest.fixture(scope="module")
def A():
    import exact_attention_flashattention_amd as A
    A._lib.load()
    return A


def f64(t):
    return t.detach().float().cpu().double().numpy()


def raw_noalloc(A, q, kc, vc, lens, S, scale, out):
    """The entry point called through the C ABI directly (ctypes, no binding logic)."""
    lib = A._lib.load()
    B, hq, d = q.shape
    _, hkv, L, _ = kc.shape
    dtype = A.ATTN_BF16 if q.dtype == torch.bfloat16 else A.ATTN_F16
    st = lib.attn_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), lens.data_ptr(), L, dtype, B, hq, hkv,
                                 d, ctypes.c_float(scale), S, out.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    assert st == 0, A._lib.STATUS_NAMES.get(st, st)
    return out


def check_against_workspace_path(A, w, q, kc, vc, lens, S, tag):
    print(f"[no-alloc] {tag}: B={q.shape[0]} hq={q.shape[1]} L={kc.shape[2]} S={S}", flush=True)
    lens_d = lens.to(DEV)
    out = torch.full_like(q, float("nan"))
    raw_noalloc(A, q, kc, vc, lens_d, 0 if S is None else S, w.scale, out)
    S_eff = A.decode_num_splits(q.shape[0], kc.shape[1], kc.shape[2]) if S is None else S
    ref_gpu = A.decode(q, kc, vc, lens_d, S_eff, w.scale)   # attn_decode_splitk + attn_merge_partials
    via_binding = A.decode_noalloc(q, kc, vc, lens_d, S, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_gpu), f"{tag}: differs from the workspace path"
    assert torch.equal(via_binding, ref_gpu), f"{tag}: binding call differs"
    ref = oracle.decode(f64(q), f64(kc), f64(vc), lens.numpy(), w.scale)
    d = np.abs(f64(out) - ref)
    print(f"[no-alloc] {tag}: max|d|={d.max():.3e} mean|d|={d.mean():.3e}", flush=True)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, tag


def test_two_calls_in_a_row_the_second_smaller(A):
    """A larger call fills more of the scratch array than the next one reads; the
    second (fewer sequences, shorter cache, other split count) must not see it."""
    q, kc, vc, lens = workloads.decode_inputs(RAG, device=DEV, batch=6, max_kv_len=9000,
                                              kv_lens=torch.tensor([9000, 1, 4097, 8191, 2048, 5000]))
    check_against_workspace_path(A, RAG, q, kc, vc, lens, None, "first call, plan's split count")
    q2, kc2, vc2, lens2 = workloads.decode_inputs(DEC, device=DEV, batch=2, max_kv_len=3000,
                                                  kv_lens=torch.tensor([3000, 700]))
    check_against_workspace_path(A, DEC, q2, kc2, vc2, lens2, 3, "second call, smaller, 3 splits")
    check_against_workspace_path(A, DEC, q2, kc2, vc2, lens2, None, "third call, same inputs, plan's count")


def test_fp16_d64_and_empty_sequences(A):
    w = workloads.Decode("noalloc_f16_d64", 3, 16, 2, 64, 1500, None, 1.0, "f16")
    q, kc, vc, lens = workloads.decode_inputs(w, device=DEV, kv_lens=torch.tensor([0, 1500, 65]), max_kv_len=1500,
                                              batch=3)
    check_against_workspace_path(A, w, q, kc, vc, lens, None, "fp16 d=64 with an empty sequence")
    out = A.decode_noalloc(q, kc, vc, lens.to(DEV), 5, w.scale)
    torch.cuda.synchronize()
    assert not out[0].float().abs().sum().item()


def test_ragged_full_size_matches_workspace_path_bit_exact(A):
    """The 64-sequence ragged decode at full size (the largest benchmarked use of the array: 34 MB of
    partial states) gives the workspace path's bits."""
    q, kc, vc, lens = workloads.decode_inputs(RAG, device=DEV)
    lens_d = lens.to(DEV)
    out = A.decode_noalloc(q, kc, vc, lens_d, None, RAG.scale)
    ref = A.decode(q, kc, vc, lens_d, None, RAG.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_too_many_splits_is_refused_before_launch(A):
    q, kc, vc, lens = workloads.decode_inputs(RAG, device=DEV, batch=64, max_kv_len=2048)
    out = torch.zeros_like(q)
    with pytest.raises(A.AttnError) as e:
        A.decode_noalloc(q, kc, vc, lens.to(DEV), 40, RAG.scale, out=out)
    assert e.value.status_name == "ATTN_ERR_SCRATCH"
    torch.cuda.synchronize()
    assert not out.float().abs().sum().item()
