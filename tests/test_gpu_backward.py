"""GPU parity of the backward pass and of the forward's log-sum-exp output.

Gradients of the plain causal (and symmetric) ALiBi forward, and of its
bias-only mitigations (clamp, log-scaled distance), against the fp64 oracle's
chain rule (oracle/backward.py, pinned to autograd and finite differences). The
pages state no tolerance for gradients; the bar used here is derived from the
arithmetic, per element:
    |gpu - o| <= 1e-2 + 1e-2 (|o| + M) + E,
with M the sum of absolute products behind the element (|dS| |K| / sqrt(d) for
dq, |dS|^T |Q| / sqrt(d) for dk, P^T |dO| for dv; oracle magnitudes). dS and P
enter the MFMAs rounded to bf16 (relative 2^-8, the unit roundoff of 8
significant bits) and P is recomputed from the forward's log-sum-exp (error up
to the bar below): errors that scale with the terms, M, not with their sum |o|;
where the terms cancel (a steep head's dq at N = 4096) they dominate. E
(parity_util.o_rounding_bound, 0 for dv) bounds the effect of the forward's
bf16 output on D = rowsum(dO O): |dD_i| <= 2^-8 sum |dO_i| |O_i| enters dS as
-P dD, and where P is nearly one-hot (log-scaled distances with a steep slope)
that is most of the error. The log-sum-exp comes from the forward's running
maximum and its row sum of bf16-rounded weights, a sum of positive terms each
within relative 2^-8, so |err| <= ln(1 + 2^-8) = 3.90e-3 plus fp32 rounding:
the bar is 4e-3 (the printed maxima stay far below it).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import F32_TOL, LSE_TOL, check_grad, check_grads, dev

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()
    return mod


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
def test_backward_small(alibi, bwd_form, B, H, N, d, causal):
    q, k, v, do = _inputs((B, H, N, d), 31)
    s = oracle.slopes_ref(H)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, torch.from_numpy(s), causal)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), causal)
    torch.cuda.synchronize()
    tag = f"B{B} H{H} N{N} d{d} causal={causal} qb={bwd_form}"
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for b in range(B):
        for h in range(H):
            check_grads((dq[b, h], dk[b, h], dv[b, h]), q[b, h], k[b, h], v[b, h], do[b, h], float(s[h]), causal,
                        f"{tag} b={b} h={h}")
    lerr = np.abs(lse.cpu().double().numpy() - oracle.lse_ref(q, k, s, causal)).max()
    print(f"[parity] lse {tag}: max err {lerr:.2e}", flush=True)
    assert lerr <= LSE_TOL


def test_backward_benchmark_shape_every_head(alibi):
    # the sequence shape of the benchmark (N = 4096, d = 128), all 16 heads of one batch
    wl = W.FWD_B8_H16_N4096_D128
    shape = (1, wl.H, wl.N, wl.d)
    q, k, v, do = _inputs(shape, wl.seed)
    s = oracle.slopes_ref(wl.H)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, torch.from_numpy(s), True)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), True)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for h in range(wl.H):
        check_grads((dq[0, h], dk[0, h], dv[0, h]), q[0, h], k[0, h], v[0, h], do[0, h], float(s[h]), True,
                    f"N4096 h={h}")


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


def test_backward_is_deterministic(alibi):
    # no atomics: two calls on the same inputs give the same bits
    q, k, v, do = _inputs((2, 4, 777, 128), 37)
    s = torch.from_numpy(oracle.slopes_ref(4))
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, s, True)
    g1 = alibi.attn_bwd(qd, kd, vd, out, dod, lse, s, True)
    g2 = alibi.attn_bwd(qd, kd, vd, out, dod, lse, s, True)
    torch.cuda.synchronize()
    for a, b, n in zip(g1, g2, ("dq", "dk", "dv")):
        assert torch.equal(a, b), n


@pytest.mark.parametrize("d", [64, 128])
def test_backward_causality_poison_bitwise(alibi, d):
    # With dO = 0 on rows >= cut, no gradient of a position < cut can depend on
    # q, k or v at positions >= cut (rows < cut see only keys < cut, and rows
    # >= cut contribute dS = P (dP - D) = 0), and every gradient at >= cut is 0.
    # Poisoning those positions must leave the first `cut` rows bit for bit.
    B, H, N, cut = 1, 4, 700, 333
    q, k, v, do = _inputs((B, H, N, d), 39)
    do[:, :, cut:] = 0
    s = torch.from_numpy(oracle.slopes_ref(H))

    def grads(q, k, v):
        qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
        out, lse = alibi.attn_fwd_train(qd, kd, vd, s, True)
        g = alibi.attn_bwd(qd, kd, vd, out, dod, lse, s, True)
        torch.cuda.synchronize()
        return [x.cpu() for x in g]

    g1 = grads(q, k, v)
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, :, cut:] = (4.0 * q[:, :, cut:].float()).to(torch.bfloat16)
    k2[:, :, cut:] = (30.0 * q[:, :, cut:].float()).to(torch.bfloat16)
    v2[:, :, cut:] = 1e4
    g2 = grads(q2, k2, v2)
    for a, b, n in zip(g1, g2, ("dq", "dk", "dv")):
        assert torch.equal(a[:, :, :cut], b[:, :, :cut]), n
        assert torch.count_nonzero(b[:, :, cut:]) == 0, n
        assert torch.isfinite(b.float()).all(), n


# ---- the bias-only mitigations of Sec. 3.4 (clamp, log-scaled distance) ----

MITS = [(-3.0, False), (None, True), (-2.0, True)]


def _mit_ids(x):
    c, l = x
    return f"c{int(c is not None)}l{int(l)}"


@pytest.mark.parametrize("mit", MITS, ids=_mit_ids)
@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 300, 128, True), (1, 3, 129, 64, True), (2, 2, 200, 64, False), (1, 2, 513, 128, False),
    (1, 2, 33, 128, True),
])
def test_backward_mitigations(alibi, bwd_form, mit, B, H, N, d, causal):
    clamp, logd = mit
    q, k, v, do = _inputs((B, H, N, d), 61)
    s = oracle.slopes_recipe_ref("steep", H, logd)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    out = alibi.attn_fwd_ex(qd, kd, vd, torch.from_numpy(s), causal, clamp=clamp, log_distance=logd, lse=lse)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), causal, clamp=clamp,
                                log_distance=logd)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    tag = f"{_mit_ids(mit)} B{B} H{H} N{N} d{d} causal={causal} qb={bwd_form}"
    for b in range(B):
        for h in range(H):
            check_grads((dq[b, h], dk[b, h], dv[b, h]), q[b, h], k[b, h], v[b, h], do[b, h], float(s[h]), causal,
                        f"{tag} b={b} h={h}", clamp=clamp, log_distance=logd)
    lerr = np.abs(lse.cpu().double().numpy() - oracle.lse_ref(q, k, s, causal, clamp, logd)).max()
    print(f"[parity] lse {tag}: max err {lerr:.2e}", flush=True)
    assert lerr <= LSE_TOL


# (z, clamp, log distance): small caps keep tanh far from linear, so the
# 1 - tanh^2 factor of the chain rule is tested, not approximated away
CAPS = [(2.0, None, False), (3.0, -3.0, True), (50.0, None, False)]


@pytest.mark.parametrize("cap", CAPS, ids=lambda c: f"z{c[0]:g}c{int(c[1] is not None)}l{int(c[2])}")
@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 300, 128, True), (1, 3, 129, 64, True), (2, 2, 200, 64, False), (1, 2, 513, 128, False),
])
def test_backward_softcap(alibi, bwd_form, cap, B, H, N, d, causal):
    z, clamp, logd = cap
    q, k, v, do = _inputs((B, H, N, d), 63)
    s = oracle.slopes_recipe_ref("steep", H, logd)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    out = alibi.attn_fwd_ex(qd, kd, vd, torch.from_numpy(s), causal, clamp=clamp, log_distance=logd, softcap=z,
                            lse=lse)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), causal, clamp=clamp,
                                log_distance=logd, softcap=z)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    tag = f"softcap z={z:g} clamp={clamp} log={logd} B{B} H{H} N{N} d{d} causal={causal} qb={bwd_form}"
    for b in range(B):
        for h in range(H):
            check_grads((dq[b, h], dk[b, h], dv[b, h]), q[b, h], k[b, h], v[b, h], do[b, h], float(s[h]), causal,
                        f"{tag} b={b} h={h}", clamp=clamp, log_distance=logd, softcap=z)
    lerr = np.abs(lse.cpu().double().numpy() - oracle.lse_ref(q, k, s, causal, clamp, logd, softcap=z)).max()
    print(f"[parity] lse {tag}: max err {lerr:.2e}", flush=True)
    assert lerr <= LSE_TOL


def test_backward_softcap_paper_settings_full_size(alibi):
    # the N = 4096, d = 128 sequence shape with the paper's cap (z = 50), floor
    # (-87) and log-scaled distances (Sec. 4.3), 4 heads of one batch, every element
    wl = W.FWD_B8_H16_N4096_D128
    H = 4
    q, k, v, do = _inputs((1, H, wl.N, wl.d), wl.seed + 5)
    s = oracle.slopes_recipe_ref("explicit", H, True)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    lse = torch.empty((1, H, wl.N), dtype=torch.float32, device="cuda")
    out = alibi.attn_fwd_ex(qd, kd, vd, torch.from_numpy(s), True, clamp=-87.0, log_distance=True, softcap=50.0,
                            lse=lse)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), True, clamp=-87.0,
                                log_distance=True, softcap=50.0)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for h in range(H):
        check_grads((dq[0, h], dk[0, h], dv[0, h]), q[0, h], k[0, h], v[0, h], do[0, h], float(s[h]), True,
                    f"N4096 cap+clamp+log h={h}", clamp=-87.0, log_distance=True, softcap=50.0)


def test_backward_mitigations_paper_settings_full_size(alibi):
    # the N = 4096, d = 128 sequence shape with the paper's floor (-87) and
    # log-scaled distances (Sec. 4.3), 8 heads of one batch, every element
    wl = W.FWD_B8_H16_N4096_D128
    H = 8
    q, k, v, do = _inputs((1, H, wl.N, wl.d), wl.seed + 3)
    s = oracle.slopes_recipe_ref("explicit", H, True)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    lse = torch.empty((1, H, wl.N), dtype=torch.float32, device="cuda")
    out = alibi.attn_fwd_ex(qd, kd, vd, torch.from_numpy(s), True, clamp=-87.0, log_distance=True, lse=lse)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), True, clamp=-87.0,
                                log_distance=True)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for h in range(H):
        check_grads((dq[0, h], dk[0, h], dv[0, h]), q[0, h], k[0, h], v[0, h], do[0, h], float(s[h]), True,
                    f"N4096 clamp+log h={h}", clamp=-87.0, log_distance=True)


def test_backward_ex_without_options_is_the_plain_backward(alibi):
    import ctypes
    q, k, v, do = (dev(x) for x in _inputs((1, 4, 300, 128), 62))
    s = alibi.slopes(4)
    out, lse = alibi.attn_fwd_train(q, k, v, s, True)
    a = alibi.attn_bwd(q, k, v, out, do, lse, s, True)
    o = alibi.FwdOpts()          # no bits set: the plain backward
    lib = alibi.load_library()
    sd = s.cuda()
    b = [torch.empty_like(q) for _ in range(3)]
    P = ctypes.c_void_p
    st = lib.alibi_attn_bwd_ex(P(q.data_ptr()), P(k.data_ptr()), P(v.data_ptr()), P(out.data_ptr()),
                               P(do.data_ptr()), P(lse.data_ptr()), P(b[0].data_ptr()), P(b[1].data_ptr()),
                               P(b[2].data_ptr()), 1, 4, 300, 128, P(sd.data_ptr()), 1, ctypes.byref(o),
                               P(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    for x, y in zip(a, b):
        assert torch.equal(x, y)
