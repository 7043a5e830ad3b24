"""Pins of the oracle's hard per-head window (oracle.variant_head_ref, window=W).

"When Attention Goes Blind", Sec. 5.2 (a steep head acts as a sliding window)
and Sec. 5.3 (a hard sliding window as the alternative to clamping, letting the
computation ignore out-of-window entries). A window of W tokens keeps key j for
query i when 0 <= i - j < W. Pinned against: the unwindowed head where the
window covers every key, the query's own value row for W = 1, zero rows for
W = 0, a brute-force loop on tiny heads (which fixes the boundary: D = W - 1 in,
D = W out), the dropped-mass bound against the unwindowed head, and the page's
88.3% out-of-window share (which the token count reproduces).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W


def _head(n_q, n_k, d, seed):
    q, k, v = W.gaussian_qkv_f32((1, 1, n_q, d), seed=seed, kv_shape=(1, 1, n_k, d))
    return q[0, 0].astype(np.float64), k[0, 0].astype(np.float64), v[0, 0].astype(np.float64)


@pytest.mark.parametrize("qo,ko", [(0, 0), (17, 0), (40, 25)])
def test_window_covering_every_key_is_the_plain_head(qo, ko):
    q, k, v = _head(23, 40, 16, 1)
    o0, w0 = oracle.variant_head_ref(q, k, v, 0.3, True, q_pos0=qo, k_pos0=ko)
    o1, w1 = oracle.variant_head_ref(q, k, v, 0.3, True, q_pos0=qo, k_pos0=ko, window=10 ** 6)
    assert np.array_equal(o0, o1) and np.array_equal(w0, w1)


def test_window_one_keeps_the_own_key():
    q, k, v = _head(30, 30, 8, 2)
    o, w = oracle.variant_head_ref(q, k, v, 0.5, True, window=1)
    assert np.array_equal(w, np.eye(30))
    assert np.array_equal(o, v)
    o, w = oracle.variant_head_ref(q, k, v, 0.5, True, window=0)
    assert np.array_equal(o, np.zeros_like(v)) and np.array_equal(w, np.zeros((30, 30)))


@pytest.mark.parametrize("win", [1, 2, 3, 6])
@pytest.mark.parametrize("m", [0.0, 0.25, 1.5])
def test_window_brute_force(win, m):
    n_q, n_k, qo = 9, 12, 3
    q, k, v = _head(n_q, n_k, 4, 3)
    o, _ = oracle.variant_head_ref(q, k, v, m, True, q_pos0=qo, window=win)
    for r in range(n_q):
        i = r + qo
        logits = {}
        for j in range(n_k):
            if 0 <= i - j < win:
                logits[j] = sum(q[r, t] * k[j, t] for t in range(4)) / 2.0 - m * (i - j)
        mx = max(logits.values())
        z = sum(math.exp(x - mx) for x in logits.values())
        for t in range(4):
            ref = sum(math.exp(x - mx) * v[j, t] for j, x in logits.items()) / z
            assert abs(o[r, t] - ref) < 1e-12


def test_window_dropped_mass_bound():
    # |out_window - out_full| <= 2 rho max|v|, rho = the full weights outside the window
    q, k, v = _head(200, 200, 32, 4)
    win = 20
    of, wf = oracle.variant_head_ref(q, k, v, 0.2, True)
    ow, _ = oracle.variant_head_ref(q, k, v, 0.2, True, window=win)
    dist = oracle.distance_ref(200, 200)
    rho = np.where(dist >= win, wf, 0.0).sum(axis=1)
    bound = 2.0 * rho[:, None] * np.abs(v).max() + 1e-12
    assert np.all(np.abs(ow - of) <= bound)
    assert rho.max() > 1e-6  # the window does cut visible weight here


def test_window_out_of_window_share_of_the_page():
    # Sec. 5.2: a steep head with an effective window of 124 tokens in a 2048
    # context leaves 88.3% of the causal entries out of window
    n, win = 2048, 124
    dist = oracle.distance_ref(n, n)
    causal = dist >= 0
    out = causal & (dist >= win)
    assert round(out.sum() / causal.sum(), 3) == 0.883


def test_window_requires_the_causal_form():
    q, k, v = _head(4, 4, 4, 5)
    with pytest.raises(ValueError):
        oracle.variant_head_ref(q, k, v, 0.1, False, window=2)


def test_window_multi_head_matches_per_head():
    q, k, v = W.gaussian_qkv_f32((2, 3, 50, 8), seed=6)
    s = oracle.slopes_ref(3)
    wins = [1, 7, 100]
    out = oracle.variant_ref(q, k, v, s, True, windows=wins)
    for b in range(2):
        for h in range(3):
            ref = oracle.variant_head_ref(q[b, h], k[b, h], v[b, h], s[h], True, window=wins[h])[0]
            assert np.array_equal(out[b, h], ref)
