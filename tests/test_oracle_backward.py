"""Pins of the oracle's gradients and row log-sum-exp (CPU only).

The gradients are tied to (i) PyTorch autograd through the forward definition
in fp64 (torch's SDPA with the explicit ALiBi bias as an additive mask, a
library routine standing in for the definition), (ii) central finite
differences of the oracle's own, separately pinned, forward (no autograd), and
(iii) closed forms the softmax fixes: the column sums of dV equal the sum of
dO, dQ vanishes when all keys are equal, and adding one vector to every key
changes no gradient. The log-sum-exp is tied to scipy and to the forward's
weights (w = exp(logit - lse)).
"""
import math

import numpy as np
import pytest

import oracle


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _torch_grads(q, k, v, do, m, causal):
    import torch
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    n = q.shape[0]
    i = torch.arange(n, dtype=torch.float64)[:, None]
    j = torch.arange(n, dtype=torch.float64)[None, :]
    bias = -m * (i - j) if causal else -m * (i - j).abs()
    if causal:
        bias = bias.masked_fill(j > i, float("-inf"))
    out = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None], attn_mask=bias)[0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("m", [0.0, 0.0625, 0.7])
def test_backward_matches_autograd(causal, m):
    n, d = 23, 16
    q, k, v, do = (_rand((n, d), s) for s in (1, 2, 3, 4))
    got = oracle.attn_backward_head_ref(q, k, v, do, m, causal)
    want = _torch_grads(q, k, v, do, m, causal)
    for g, w in zip(got, want):
        assert np.allclose(g, w, atol=1e-12, rtol=1e-10)


def test_backward_matches_finite_differences():
    n, d, m, eps = 6, 4, 0.3, 1e-6
    q, k, v, do = (_rand((n, d), s, 0.7) for s in (5, 6, 7, 8))
    dq, dk, dv = oracle.attn_backward_head_ref(q, k, v, do, m, True)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_head_ref(qq, kk, vv, m, True)
        return float(np.sum(o * do))

    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert np.allclose(grad, num, atol=1e-7), which


def test_dv_column_sum_equals_do_sum():
    q, k, v, do = (_rand((17, 8), s) for s in (9, 10, 11, 12))
    _, _, dv = oracle.attn_backward_head_ref(q, k, v, do, 0.25, True)
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)


def test_dq_vanishes_for_equal_keys_and_key_shift_changes_nothing():
    n, d = 12, 8
    q, v, do = (_rand((n, d), s) for s in (13, 14, 15))
    k_same = np.tile(_rand((1, d), 16), (n, 1))
    dq, _, _ = oracle.attn_backward_head_ref(q, k_same, v, do, 0.5, True)
    assert np.allclose(dq, 0.0, atol=1e-12)
    k = _rand((n, d), 17)
    g1 = oracle.attn_backward_head_ref(q, k, v, do, 0.5, True)
    g2 = oracle.attn_backward_head_ref(q, k + _rand((1, d), 18), v, do, 0.5, True)
    for a, b in zip(g1, g2):
        assert np.allclose(a, b, atol=1e-11)


def test_lse_against_scipy_and_weights():
    from scipy.special import logsumexp
    n, d, m = 20, 8, 0.4
    q, k, v = (_rand((n, d), s) for s in (19, 20, 21))
    lse = oracle.lse_head_ref(q, k, m, True)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    logits = np.where(j <= i, q @ k.T / math.sqrt(d) - m * (i - j), -np.inf)
    assert np.allclose(lse, logsumexp(logits, axis=1), atol=1e-12)
    _, w = oracle.attn_head_ref(q, k, v, m, True)
    assert np.allclose(np.where(j <= i, np.exp(logits - lse[:, None]), 0.0), w, atol=1e-13)


def test_backward_magnitudes_bound_the_gradients():
    # |sum_j a_j b_j| <= sum_j |a_j| |b_j|: each magnitude bounds its gradient,
    # with equality where no terms cancel (all of one sign: dv with do >= 0)
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((24, 8)) for _ in range(3))
    do = rng.standard_normal((24, 8))
    for causal in (True, False):
        (dq, dk, dv), (mq, mk, mv) = oracle.attn_backward_head_ref(q, k, v, do, 0.3, causal, magnitudes=True)
        assert np.all(np.abs(dq) <= mq * (1 + 1e-12)) and np.all(np.abs(dk) <= mk * (1 + 1e-12))
        assert np.all(np.abs(dv) <= mv * (1 + 1e-12))
        plain = oracle.attn_backward_head_ref(q, k, v, do, 0.3, causal)
        for a, b in zip(plain, (dq, dk, dv)):
            assert np.array_equal(a, b)
    (_, _, dv), (_, _, mv) = oracle.attn_backward_head_ref(q, k, v, np.abs(do), 0.3, True, magnitudes=True)
    assert np.allclose(dv, mv, rtol=1e-13)


# ---- the bias-only mitigations (clamp, log-scaled distance) in the backward ----

def _torch_grads_bias(q, k, v, do, bias):
    import torch
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt[None], kt[None], vt[None],
                                                           attn_mask=torch.tensor(bias))[0]
    out.backward(torch.tensor(do, dtype=torch.float64))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("clamp,logd", [(-2.0, False), (None, True), (-1.5, True)])
def test_backward_mitigations_match_autograd(causal, clamp, logd):
    # autograd through SDPA with the mitigation's additive bias, whose values are
    # the forward oracle's own (oracle.variant_head_ref's weights are pinned there)
    n, d, m = 21, 16, 0.6
    q, k, v, do = (_rand((n, d), s) for s in (31, 32, 33, 34))
    _, w = oracle.variant_head_ref(q, k, v, m, causal, clamp, logd)
    a = q @ k.T / math.sqrt(d)
    lse = oracle.lse_head_ref(q, k, m, causal, clamp, logd)
    # logits recovered from the pinned weights: log w + lse, -inf where w = 0 under the mask
    with np.errstate(divide="ignore"):
        logits = np.log(w) + lse[:, None]
    bias = logits - a
    got = oracle.attn_backward_head_ref(q, k, v, do, m, causal, clamp=clamp, log_distance=logd)
    want = _torch_grads_bias(q, k, v, do, bias)
    for g, x in zip(got, want):
        assert np.allclose(g, x, atol=1e-11, rtol=1e-9)


@pytest.mark.parametrize("clamp,logd", [(-2.0, False), (None, True), (-1.0, True)])
def test_backward_mitigations_match_finite_differences(clamp, logd):
    n, d, m, eps = 6, 4, 0.8, 1e-6
    q, k, v, do = (_rand((n, d), s, 0.7) for s in (35, 36, 37, 38))
    dq, dk, dv = oracle.attn_backward_head_ref(q, k, v, do, m, True, clamp=clamp, log_distance=logd)

    def loss(qq, kk, vv):
        o, _ = oracle.variant_head_ref(qq, kk, vv, m, True, clamp, logd)
        return float(np.sum(o * do))

    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert np.allclose(grad, num, atol=1e-7), which


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("z,clamp,logd", [(2.0, None, False), (1.5, -2.0, True), (4.0, None, True)])
def test_backward_softcap_matches_autograd(causal, z, clamp, logd):
    # autograd through z tanh(q k / sqrt(d) / z) plus a constant bias; the
    # bias is what the pinned forward oracle's weights leave once its capped
    # content logits are taken away (log w + lse - z tanh(A / z)). Small z
    # keeps tanh well away from linear, so a missing or wrong 1 - tanh^2
    # factor fails.
    import torch
    n, d, m = 19, 16, 0.5
    q, k, v, do = (_rand((n, d), s, 1.5) for s in (51, 52, 53, 54))
    _, w = oracle.variant_head_ref(q, k, v, m, causal, clamp, logd, softcap=z)
    lse = oracle.lse_head_ref(q, k, m, causal, clamp, logd, softcap=z)
    a = q @ k.T / math.sqrt(d)
    with np.errstate(divide="ignore"):
        bias = np.log(w) + lse[:, None] - z * np.tanh(a / z)
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    logits = z * torch.tanh(qt @ kt.T / math.sqrt(d) / z) + torch.tensor(bias)
    out = torch.softmax(logits, dim=-1) @ vt
    out.backward(torch.tensor(do, dtype=torch.float64))
    got = oracle.attn_backward_head_ref(q, k, v, do, m, causal, clamp=clamp, log_distance=logd, softcap=z)
    for g, x in zip(got, (qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy())):
        assert np.allclose(g, x, atol=1e-11, rtol=1e-9)


@pytest.mark.parametrize("z,logd", [(1.0, False), (2.5, True)])
def test_backward_softcap_matches_finite_differences(z, logd):
    n, d, m, eps = 6, 4, 0.8, 1e-6
    q, k, v, do = (_rand((n, d), s, 1.2) for s in (55, 56, 57, 58))
    dq, dk, dv = oracle.attn_backward_head_ref(q, k, v, do, m, True, log_distance=logd, softcap=z)

    def loss(qq, kk, vv):
        o, _ = oracle.variant_head_ref(qq, kk, vv, m, True, None, logd, softcap=z)
        return float(np.sum(o * do))

    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            num[idx] = (loss(*plus) - loss(*minus)) / (2 * eps)
        assert np.allclose(grad, num, atol=1e-7), which


def test_backward_large_softcap_is_the_uncapped_head():
    # z tanh(A / z) = A - A^3 / (3 z^2) + ...: at z = 1e6 the capped gradients
    # agree with the plain ones to ~1e-12 relative
    q, k, v, do = (_rand((17, 8), s) for s in (59, 60, 61, 62))
    for causal in (True, False):
        got = oracle.attn_backward_head_ref(q, k, v, do, 0.3, causal, softcap=1e6)
        want = oracle.attn_backward_head_ref(q, k, v, do, 0.3, causal)
        for g, x in zip(got, want):
            assert np.allclose(g, x, atol=1e-9, rtol=1e-9)


def test_backward_clamp_above_every_bias_is_the_slope_free_head():
    # a floor at 0 lifts every bias -m D <= 0 to 0: the gradients of m = 0
    q, k, v, do = (_rand((15, 8), s) for s in (39, 40, 41, 42))
    for causal in (True, False):
        got = oracle.attn_backward_head_ref(q, k, v, do, 0.9, causal, clamp=0.0)
        want = oracle.attn_backward_head_ref(q, k, v, do, 0.0, causal)
        for g, x in zip(got, want):
            assert np.allclose(g, x, atol=1e-13)


@pytest.mark.parametrize("case", ["steep_log", "plain"])
def test_output_rounding_bound_covers_its_effect(case):
    # The GPU gradient bar carries a term E for the forward's bf16 output: the
    # backward forms D = rowsum(dO O) from the stored O. Here O is rounded to
    # bf16 (torch's round-to-nearest-even) on the CPU and the chain rule redone
    # in fp64 with that D: the change in dq and dk stays within E everywhere.
    # The steep log-distance head (m = 14 on ln(D + 1), 300 tokens, d = 128) is
    # where the rest of the bar alone is exceeded: P is nearly one-hot there.
    import torch
    import workloads as W
    from parity_util import o_rounding_bound
    if case == "steep_log":
        q, k, v = (x[0, 1].double().numpy() for x in W.gaussian_qkv_bf16((1, 2, 300, 128), seed=61))
        do = W.to_bf16_tensor(W.gaussian_f32((1, 2, 300, 128), 161))[0, 1].double().numpy()
        m, logd = float(oracle.slopes_recipe_ref("steep", 2, True)[1]), True
    else:
        q, k, v, do = (_rand((200, 64), s) for s in (43, 44, 45, 46))
        m, logd = 0.25, False
    o, p = oracle.variant_head_ref(q, k, v, m, True, log_distance=logd)
    (rq, rk, _), (mq, _, _) = oracle.attn_backward_head_ref(q, k, v, do, m, True, magnitudes=True,
                                                            log_distance=logd)
    ob = torch.from_numpy(o).to(torch.bfloat16).double().numpy()
    scale = 1.0 / math.sqrt(q.shape[1])
    ds = p * (do @ v.T - np.sum(do * ob, axis=-1, keepdims=True))
    eq, ek = o_rounding_bound(p, o, q, k, do)
    for got, ref, e in ((ds @ k * scale, rq, eq), (ds.T @ q * scale, rk, ek)):
        err = np.abs(got - ref)
        assert np.all(err <= e * (1 + 1e-9) + 1e-15)
    if case == "steep_log":
        err_q = np.abs(ds @ k * scale - rq)
        assert np.any(err_q > 1e-2 + 1e-2 * (np.abs(rq) + mq))
