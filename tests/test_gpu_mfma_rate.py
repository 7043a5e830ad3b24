"""The measurement-only MFMA-rate kernel runs every MFMA it is timed for.

It is the sustained matrix rate that the forward's MFMA rate is read against
beside the datasheet peak, so the test checks that each wave really performed
iters rounds of the four accumulator chains on the given operands: the sum of
a product's elements is sum_k colsum(A)[k] rowsum(B)[k] whatever the
accumulator layout, and with operands in {-1, 0, 1} every partial sum is an
integer below 2^24, so the check is exact.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("valu", [0, 1], ids=["mfma", "mfma+valu"])
@pytest.mark.parametrize("iters,workgroups", [(1, 1), (8, 3), (5, 300)])
def test_mfma_rate_runs_every_chain(iters, workgroups, valu):
    import alibi_linear_position_amd as alibi
    lib = alibi.load_library()
    rng = np.random.default_rng(1000 * iters + workgroups)
    frags = rng.integers(-1, 2, size=(8, 64, 8)).astype(np.float32)   # A_0..A_3, B_0..B_3; lane, element
    dev = torch.from_numpy(frags).to(torch.bfloat16).cuda().contiguous()
    sink = torch.full((8 * workgroups,), float("nan"), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.alibi_debug_mfma_rate(dev.data_ptr(), iters, valu, sink.data_ptr(), workgroups, st) == 0
    torch.cuda.synchronize()
    # k = 8 (lane // 32) + element for both operands: per half h, the sums over
    # rows of A (columns of B) are the lane sums over that half
    F = frags.reshape(8, 2, 32, 8).sum(axis=2)   # [fragment, half, element]
    want = iters * sum(float(np.sum(F[c] * F[4 + m])) for c in range(4) for m in range(4))
    got = sink.cpu().numpy()
    print(f"[parity] mfma rate valu={valu} iters={iters} workgroups={workgroups}: {got[:3]} vs {want}", flush=True)
    assert np.all(got == want)
