"""GPU parity of the backward pass and of the forward's log-sum-exp output.

Gradients of the plain causal (and symmetric) ALiBi forward against the fp64
oracle's chain rule (oracle/backward.py, pinned to autograd and finite
differences). The pages state no tolerance for gradients; the bar used here is
|gpu - o| <= 1e-2 + 1e-2 |o| per element: the bf16 output rounding alone is
2^-9 |o|, and P and dS enter the MFMAs as bf16. The log-sum-exp comes from the
forward's running maximum and its row sum of bf16-rounded weights, whose
relative error is at most 2^-9 (a sum of positive terms), so |err| <= ln(1 +
2^-9) = 1.95e-3 plus fp32 rounding: the bar is 2.5e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import F32_TOL, dev

pytestmark = pytest.mark.gpu

G_ATOL = 1e-2
G_RTOL = 1e-2
LSE_TOL = 2.5e-3


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()
    return mod


def check_grad(gpu, ref, label):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    err = np.abs(g - ref)
    bad = int(np.sum(err > G_ATOL + G_RTOL * np.abs(ref)))
    print(f"[parity] {label}: max|err|={err.max():.3e} max|ref|={np.abs(ref).max():.3e} failing={bad}",
          flush=True)
    assert np.all(np.isfinite(g)) and bad == 0, label


def _inputs(shape, seed):
    q, k, v = W.gaussian_qkv_bf16(shape, seed=seed)
    do = W.to_bf16_tensor(W.gaussian_f32(shape, seed + 100))
    return q, k, v, do


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 33, 64, True), (1, 2, 100, 64, False), (2, 3, 300, 128, True),
    (1, 4, 1000, 64, True), (1, 2, 513, 128, False), (2, 2, 200, 128, True),
    # a key block with a single query tile (N = 129: keys 128.. see one 32-row tile),
    # shorter than one tile, a single token, and a non-causal multi-tile d = 128 case
    (1, 2, 129, 128, True), (1, 3, 16, 64, True), (1, 2, 1, 128, True), (2, 2, 160, 128, False),
])
def test_backward_small(alibi, B, H, N, d, causal):
    q, k, v, do = _inputs((B, H, N, d), 31)
    s = oracle.slopes_ref(H)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, torch.from_numpy(s), causal)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), causal)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attn_backward_ref(q, k, v, do, s, causal)
    tag = f"B{B} H{H} N{N} d{d} causal={causal}"
    check_grad(dq, rq, "dq " + tag)
    check_grad(dk, rk, "dk " + tag)
    check_grad(dv, rv, "dv " + tag)
    lerr = np.abs(lse.cpu().double().numpy() - oracle.lse_ref(q, k, s, causal)).max()
    print(f"[parity] lse {tag}: max err {lerr:.2e}", flush=True)
    assert lerr <= LSE_TOL


def test_backward_full_size_two_heads(alibi):
    wl = W.FWD_B8_H16_N4096_D128
    shape = (1, wl.H, wl.N, wl.d)
    q, k, v, do = _inputs(shape, wl.seed)
    s = oracle.slopes_ref(wl.H)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, torch.from_numpy(s), True)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), True)
    torch.cuda.synchronize()
    for h in (0, wl.H - 1):
        rq, rk, rv = oracle.attn_backward_head_ref(q[0, h], k[0, h], v[0, h], do[0, h], float(s[h]), True)
        check_grad(dq[0, h], rq, f"dq N4096 h={h}")
        check_grad(dk[0, h], rk, f"dk N4096 h={h}")
        check_grad(dv[0, h], rv, f"dv N4096 h={h}")


def test_forward_with_lse_is_the_same_forward(alibi):
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((2, 4, 333, 128), seed=33))
    s = alibi.slopes(4)
    a = alibi.attn_fwd(q, k, v, s, causal=True)
    b, lse = alibi.attn_fwd_train(q, k, v, s, True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_lse_fp32_generic(alibi):
    q, k, v = W.gaussian_qkv_f32((1, 3, 45, 24), seed=34)
    s = oracle.slopes_ref(3)
    lse = torch.empty((1, 3, 45), dtype=torch.float32, device="cuda")
    alibi.attn_fwd_ex(dev(torch.from_numpy(q)), dev(torch.from_numpy(k)), dev(torch.from_numpy(v)),
                      torch.from_numpy(s), True, lse=lse)
    torch.cuda.synchronize()
    err = np.abs(lse.cpu().double().numpy() - oracle.lse_ref(q, k, s, True)).max()
    print(f"[parity] fp32 lse: max err {err:.2e}", flush=True)
    assert err <= F32_TOL


def test_backward_zero_slopes_match_torch(alibi):
    # m = 0: the gradients of causal SDPA, by torch autograd in fp32 on the CPU
    q, k, v, do = _inputs((1, 2, 150, 64), 35)
    z = torch.zeros(2, dtype=torch.float32)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, z, True)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, z, True)
    torch.cuda.synchronize()
    qt, kt, vt = (x.float().requires_grad_(True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
    o.backward(do.float())
    for g, r, n in ((dq, qt.grad, "dq"), (dk, kt.grad, "dk"), (dv, vt.grad, "dv")):
        check_grad(g, r.double().numpy(), f"{n} zero slopes vs torch")
