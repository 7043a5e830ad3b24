"""Every element of the large configurations against the fp64 oracle (needs an MI355X).

The 16384-token forward (B1 H16 d128), the N = 4096, d = 128 forward the
benchmark times (B8 H16) and the 32768-token decode (B32 H32 d128) are compared
element by element, one (b, h) at a time so that the oracle's (N, N) matrices
stay within host memory (the backward at the benchmark's sequence shape,
B1 H16 N4096 d128, is compared the same way in test_gpu_backward.py). The kernels run in the launch configuration bench.py times (the
library's automatic choice). Tolerances as in tests/parity_util.py and
tests/test_gpu_backward.py.
"""
import time

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Bf16Stats, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()
    return mod


@pytest.mark.parametrize("wl", [W.FWD_B1_H16_N16384_D128, W.FWD_B8_H16_N4096_D128], ids=lambda w: w.name)
def test_fwd_every_element(alibi, wl):
    q, k, v = W.gaussian_qkv_bf16(wl.shape, seed=wl.seed)
    out = alibi.attn_fwd(dev(q), dev(k), dev(v), alibi.slopes(wl.H), causal=True).cpu()
    s = oracle.slopes_ref(wl.H)
    st = Bf16Stats(wl.name)
    t0 = time.perf_counter()
    for b in range(wl.B):
        for h in range(wl.H):
            ref, _ = oracle.attn_head_ref(q[b, h], k[b, h], v[b, h], float(s[h]), causal=True)
            st.add(out[b, h], ref)
        print(f"[parity] {wl.name}: batch {b} done, {time.perf_counter() - t0:.1f} s", flush=True)
    st.finish()


def test_decode_every_element(alibi):
    wl = W.DECODE_B32_H32_L32768_D128
    kc = W.device_gaussian_bf16((wl.B, wl.H, wl.L, wl.d), seed=wl.seed)
    vc = W.device_gaussian_bf16((wl.B, wl.H, wl.L, wl.d), seed=wl.seed + 1)
    q = W.device_gaussian_bf16((wl.B, wl.H, wl.d), seed=wl.seed + 2)
    out = alibi.attn_decode(q, kc, vc, alibi.slopes(wl.H)).cpu()
    s = oracle.slopes_ref(wl.H)
    qh = q.cpu()
    st = Bf16Stats(wl.name)
    t0 = time.perf_counter()
    for b in range(wl.B):  # one batch of caches on the host at a time (2 x 256 MB)
        kb, vb = kc[b:b + 1].cpu(), vc[b:b + 1].cpu()
        st.add(out[b:b + 1], oracle.decode_ref(qh[b:b + 1], kb, vb, s))
        if b % 8 == 7:
            print(f"[parity] {wl.name}: batch {b} done, {time.perf_counter() - t0:.1f} s", flush=True)
    st.finish()
    del kc, vc
    torch.cuda.empty_cache()
