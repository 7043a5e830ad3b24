"""Pins of the oracle's underflow diagnostics (CPU only).

Printed values from "When Attention Goes Blind: Numerical Failure in ALiBi
Positional Encodings" (App. A Table 4, Table 1, App. F Table 8, Sec. 3.3,
Sec. 3.4, Sec. 5.2), stored under tests/golden/underflow_tables.json.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    with open(os.path.join(GOLDEN, "underflow_tables.json")) as f:
        return json.load(f)


def test_thresholds_table4():
    g = _g()["table4"]
    for fmt in ("bf16", "fp32"):
        t = oracle.format_thresholds(fmt)
        for key in ("tau_u", "tau_d", "tau_o"):
            assert round(t[key], g["decimals"]) == g[fmt][key], (fmt, key)
    # closed forms behind the table
    assert oracle.format_thresholds("bf16")["tau_u"] == pytest.approx(-133 * math.log(2), rel=1e-15)
    assert oracle.format_thresholds("fp32")["tau_u"] == pytest.approx(-149 * math.log(2), rel=1e-15)


def test_blindness_distance_definition_bruteforce():
    # Delta(eps) = least natural d with eps - m d <= tau, found by plain search
    for m in (0.70710678, 0.25, 0.0039, 1.0):
        for eps in (0.0, 3.5, -2.0):
            for tau in (-87.3365, -92.1886):
                d = 0
                while eps - m * d > tau:
                    d += 1
                assert oracle.blindness_distance(m, eps, tau) == d


def test_share_at_distance_2048_sixteen_heads():
    g = _g()
    tau_d = oracle.format_thresholds("bf16")["tau_d"]
    s = oracle.slopes_ref(16).astype(np.float64)
    share = oracle.underflow_fraction_by_distance(s, 2048, tau_d)
    assert round(share, 3) == g["sec33_share_at_distance_2048_16_heads"]


def test_steep_window_share():
    g = _g()
    tau_d = oracle.format_thresholds("bf16")["tau_d"]
    s0 = float(oracle.slopes_ref(16)[0])
    assert round(oracle.expected_blindness_distance(s0, tau_d)) == 124
    share = oracle.underflow_fraction_causal(s0, 2048, tau_d)
    assert round(share, 3) == g["sec52_steep_window_124_context_2048_share"]
    # brute force over the triangle
    n = 300
    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    tri = j <= i
    bf = np.sum((-s0 * (i - j) <= tau_d) & tri) / np.sum(tri)
    assert oracle.underflow_fraction_causal(s0, n, tau_d) == pytest.approx(bf, rel=1e-14)


def test_log_scaled_blindness():
    g = _g()
    tau_d = oracle.format_thresholds("bf16")["tau_d"]
    s0 = float(oracle.slopes_ref(16)[0])
    got = oracle.log_scaled_blindness_distance(s0, tau_d)
    assert got == pytest.approx(g["sec34_log_scaled_delta_1_16_heads"], rel=5e-3)


def test_data_share_reduces_to_analytic_when_content_is_zero():
    n, m = 400, 0.5
    q = np.zeros((n, 8))
    k = np.random.default_rng(0).standard_normal((n, 8))
    tau = oracle.format_thresholds("bf16")["tau_u"]
    got = oracle.underflow_fraction_data(q, k, m, tau)
    assert got["share"] == pytest.approx(oracle.underflow_fraction_causal(m, n, tau), rel=1e-14)
    # last row: distances 0..n-1, share of those with -m d <= tau
    want_last = np.mean(-m * np.arange(n) <= tau)
    assert got["last_row_share"] == pytest.approx(want_last, rel=1e-14)


def test_data_share_row_maximum_off_the_diagonal_closed_form():
    # Table 4's condition is on the stable-softmax exponent x_ij = s_ij - max_j s_ij.
    # Key 0 is aligned with every query and scores far above the rest, so each
    # row's maximum sits at distance i, not on the diagonal: with d = 4,
    # q_i = (400, 0, 0, 0), k_0 = (1, 0, 0, 0) and k_j = (0, 1, 0, 0) for j >= 1,
    # s_i0 = 400 / 2 - m i and s_ij = -m (i - j). With m = 1 and N = 100 the
    # maximum is s_i0 = 200 - i >= 101 and every other entry has
    # x_ij = j - 200 <= -101 < tau_u(bf16) = -92.19: all of them underflow,
    # i.e. N (N - 1) / 2 of the N (N + 1) / 2 causal entries and N - 1 of the
    # last row's N. (Without the maximum, only entries with i - j >= 93 would.)
    n, m = 100, 1.0
    q = np.zeros((n, 4))
    q[:, 0] = 400.0
    k = np.zeros((n, 4))
    k[0, 0] = 1.0
    k[1:, 1] = 1.0
    tau = oracle.format_thresholds("bf16")["tau_u"]
    got = oracle.underflow_fraction_data(q, k, m, tau)
    assert got["share"] == pytest.approx((n - 1) / (n + 1), rel=1e-15)
    assert got["last_row_share"] == pytest.approx((n - 1) / n, rel=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_data_share_bruteforce_python_loops(seed):
    # Tiny heads with large content scores (so row maxima move off the
    # diagonal), counted with plain Python loops: score, row maximum over the
    # visible keys, exponent, threshold.
    rng = np.random.default_rng(seed)
    n, d = 14, 3
    q = rng.standard_normal((n, d)) * 30.0
    k = rng.standard_normal((n, d))
    m, tau = 0.9, -20.0
    for causal in (True, False):
        hit = tot = 0
        last = 0.0
        for i in range(n):
            keys = range(i + 1) if causal else range(n)
            s = []
            for j in keys:
                dot = 0.0
                for t in range(d):
                    dot += float(q[i, t]) * float(k[j, t])
                s.append(dot / math.sqrt(d) - m * abs(i - j))
            top = max(s)
            h = sum(1 for x in s if x - top <= tau)
            hit += h
            tot += len(s)
            last = h / len(s)
        got = oracle.underflow_fraction_data(q, k, m, tau, causal=causal)
        assert got["share"] == pytest.approx(hit / tot, rel=1e-12), causal
        assert got["last_row_share"] == pytest.approx(last, rel=1e-12), causal
        assert 0 < hit < tot  # the case exercises both sides of the threshold


def test_data_share_several_thresholds_in_one_pass():
    rng = np.random.default_rng(5)
    q, k = rng.standard_normal((40, 8)) * 6.0, rng.standard_normal((40, 8))
    taus = [-10.0, -30.0, -92.0]
    many = oracle.underflow_fraction_data(q, k, 0.7, taus)
    for t, r in zip(taus, many):
        assert r == oracle.underflow_fraction_data(q, k, 0.7, t)
