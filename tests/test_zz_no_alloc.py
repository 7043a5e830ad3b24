"""The decode entry point that allocates nothing, against the ordinary decode (needs an MI355X).

alibi_attn_decode_noalloc keeps its partial states in the library's per-device
scratch array instead of an allocated workspace. Two calls in a row, the second
with a smaller input (so a stale first-call state in the shared scratch would
show), must give the bitwise output of alibi_attn_decode and match the fp64
oracle within the bf16 bar.
"""
import pytest
import torch

import oracle
import workloads as W
from parity_util import check_bf16, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()
    return mod


def test_noalloc_decode_matches_decode_on_two_calls(alibi):
    shapes = [(4, 8, 20000, 128, 81), (2, 3, 700, 64, 82)]  # the second smaller
    for B, H, L, d, seed in shapes:
        q, kc, vc = W.gaussian_qkv_bf16((B, H, d), seed=seed, kv_shape=(B, H, L, d))
        qd, kd, vd = dev(q), dev(kc), dev(vc)
        s = alibi.slopes(H).cuda()
        assert alibi.decode_ws_bytes(B, H, L, d) > 0  # both shapes use the scratch
        ref_call = alibi.attn_decode(qd, kd, vd, s)
        out = torch.empty_like(qd)
        got = alibi.attn_decode_noalloc(qd, kd, vd, s, out)
        torch.cuda.synchronize()
        print(f"[parity] noalloc decode B{B} H{H} L{L} d{d}: bitwise equal = {torch.equal(got, ref_call)}",
              flush=True)
        assert torch.equal(got, ref_call)
        check_bf16(got, oracle.decode_ref(q, kc, vc, oracle.slopes_ref(H)), f"noalloc decode B{B} H{H} L{L} d{d}")
