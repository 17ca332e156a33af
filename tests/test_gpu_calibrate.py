"""GPU checks of the measurement helpers (include/attn_calibrate.h), called
through the C ABI.  They are not part of the attention path; the bench quotes
kernel rates against what they measure, so what they compute is pinned here.
"""

import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    from exact_attention_flashattention_amd import _lib
    return _lib.load()


def bf16(x):
    return float(torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).float())


def test_mfma_loop_computes_its_chains(lib):
    # Each wave runs `iters` rounds of four identical 32x32x16 chains, A from the
    # lanes' thread indices and B constant.  Summed over a wave's 64 lanes and
    # 16 accumulators, every output element appears once, so the total is
    # 4 · iters · sum_k (column k of A summed) · (row k of B summed): lanes
    # 32h .. 32h+31 hold k = 8h .. 8h+7, word i of a lane holding k = 8h+2i, 8h+2i+1.
    blocks, iters = 3, 8
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    assert lib.attn_calib_mfma_bf16(out.data_ptr(), blocks, iters, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.double().cpu().view(blocks, 4, 64).sum(dim=2)
    for w in range(4):
        total = 0.0
        for h in range(2):
            for i in range(4):
                col_even = sum(bf16((64 * w + 32 * h + r + i) * 1e-3) for r in range(32))  # A[., 8h+2i]
                col_odd = 32 * 0.5                                                         # A[., 8h+2i+1]
                total += col_even * 32 * bf16(0.25) + col_odd * 32 * bf16(0.01 * i)
        expect = 4 * iters * total
        for b in range(blocks):
            assert abs(got[b, w].item() - expect) <= 1e-5 * abs(expect), (b, w, got[b, w].item(), expect)


def test_streaming_read_reads_and_writes_nothing(lib):
    buf = torch.ones(1 << 20, dtype=torch.float32, device="cuda")
    scratch = torch.full((4096,), 7, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    assert lib.attn_calib_read(buf.data_ptr(), buf.numel() * 4, scratch.data_ptr(), 64, stream.cuda_stream) == 0
    torch.cuda.synchronize()
    # every 16-byte chunk is four equal words, whose XOR is 0: the store never happens
    assert torch.all(scratch == 7)
