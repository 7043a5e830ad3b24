"""Pins of the fp64 oracle to what the pages and the mathematics fix (CPU only).

Each test ties one oracle function to something other than itself: values the
pages print (fixtures under tests/golden/, each with its citation), closed
forms, invariants, special cases that reduce to a library routine (torch's
scaled_dot_product_attention in fp64, scipy's softmax), and brute force on tiny
inputs. A plausible slip in the oracle (a dropped scale, a wrong sign of the
bias, j - i instead of i - j, a transposed operand, a missing mask, a sorted
slope list) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st
from scipy.special import softmax as scipy_softmax

import oracle
from workloads import tiny_example_qkv_f64, tiny_example_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- slopes ----

def test_slopes_printed_lists_bitwise():
    g = _golden("slopes_printed.json")
    for key in ("H4", "H6", "H8"):
        H = int(key[1:])
        got = oracle.slopes_ref(H)
        assert got.dtype == np.float32
        assert got.tolist() == [np.float32(x) for x in g[key]], key


def test_slopes_ratio_power_of_two():
    for H in (1, 2, 4, 8, 16, 32, 64, 128):
        s = oracle.slopes_pow2_ref(H)
        assert s[0] == pytest.approx(2.0 ** (-8.0 / H), rel=1e-15)
        assert np.allclose(s[1:] / s[:-1], 2.0 ** (-8.0 / H), rtol=1e-13, atol=0)
        assert s[-1] == 2.0 ** -8  # every schedule ends at 2^-8


def test_slopes_non_power_of_two_structure():
    # the c-schedule first, then even entries of the 2c schedule, unsorted
    for H in (3, 5, 6, 7, 9, 12, 20, 40, 56, 71, 112):
        c = 1 << (H.bit_length() - 1)
        s = oracle.slopes_ref(H).astype(np.float64)
        base = np.array([2.0 ** (-8.0 * (h + 1) / c) for h in range(c)]).astype(np.float32)
        dbl = np.array([2.0 ** (-8.0 * (h + 1) / (2 * c)) for h in range(2 * c)]).astype(np.float32)
        assert np.array_equal(s[:c], base)
        assert np.array_equal(s[c:], dbl[0:2 * (H - c):2])
        assert len(set(s.tolist())) == H


def test_slopes_table8_default_row_nine_heads():
    # Table 8's default row is recovered only by the unsorted non-power-of-two rule.
    g = _golden("underflow_tables.json")
    tau_d = oracle.format_thresholds("bf16")["tau_d"]
    s = sorted(oracle.slopes_ref(9).astype(np.float64), reverse=True)
    got = [round(oracle.expected_blindness_distance(m, tau_d)) for m in s]
    assert got == g["table8_default_9_heads"]


def test_slopes_table1_blindness():
    g = _golden("underflow_tables.json")["table1"]
    tau_d = oracle.format_thresholds("bf16")["tau_d"]
    for row in g.values():
        s = oracle.slopes_ref(row["H"]).astype(np.float64)
        assert round(oracle.expected_blindness_distance(s[0], tau_d)) == row["delta_1"]
        assert round(oracle.expected_blindness_distance(s[-1], tau_d)) == row["delta_H"]


def test_slopes_twelve_heads_values():
    # 12 heads: the 8-head schedule then entries 0, 2, 4, 6 of the 16-head schedule
    s = oracle.slopes_ref(12).astype(np.float64)
    want = [2.0 ** -e for e in (1, 2, 3, 4, 5, 6, 7, 8)] + [2.0 ** -e for e in (0.5, 1.5, 2.5, 3.5)]
    assert np.array_equal(s, np.array(want, dtype=np.float32).astype(np.float64))


# ---------------------------------------------------------- bias values ----

def test_bias_worked_values():
    g = _golden("worked_values.json")
    p = g["pair"]
    b = oracle.bias_ref(p["m"], oracle.distance_ref(1, 1, p["i"], p["j"]), causal=True)[0, 0]
    assert b == p["bias"]
    assert p["content"] + b == p["logit"]
    for e in g["extrapolation"]:
        b = oracle.bias_ref(e["m"], oracle.distance_ref(1, 1, e["dist"], 0), True)[0, 0]
        assert b == e["bias"]  # exact in binary
    for e in g["quantmemo"]:
        b = oracle.bias_ref(e["m"], oracle.distance_ref(1, 1, e["i"], e["j"]), False)[0, 0]
        assert e["content"] + b == pytest.approx(e["score"], abs=1e-12)
    pr = g["practice"]
    b = oracle.bias_ref(pr["m"], oracle.distance_ref(1, 1, pr["dist"], 0), False)[0, 0]
    assert pr["content"] + b == pytest.approx(pr["score"], abs=1e-12)


def test_bias_translation_asserts():
    g = _golden("worked_values.json")["devto_asserts"]
    b = oracle.bias_ref(g["m"], oracle.distance_ref(g["N"], g["N"]), causal=True)
    (i1, j1), (i2, j2) = g["equal_pairs"]
    assert b[i1, j1] == b[i2, j2]
    assert b[tuple(g["zero_at"])] == 0.0
    # the bias falls to the left of the diagonal (older keys pay more)
    assert b[7, 0] < b[7, 6] < b[7, 7]


def test_bias_symmetric_when_not_causal():
    d = oracle.distance_ref(9, 9)
    b = oracle.bias_ref(0.5, d, causal=False)
    assert np.array_equal(b, b.T)
    assert b[2, 7] == -2.5 and b[7, 2] == -2.5


def test_distance_positions_offsets():
    d = oracle.distance_ref(1, 5, q_pos0=4, k_pos0=0)
    assert d.tolist() == [[4, 3, 2, 1, 0]]


# -------------------------------------------------------------- softmax ----

def test_softmax_rows_against_scipy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 11)) * 30
    x[2, 5:] = -np.inf
    assert np.allclose(oracle.softmax_rows_ref(x), scipy_softmax(x, axis=-1), rtol=1e-14, atol=0)
    y = np.full((2, 3), -np.inf)
    assert np.array_equal(oracle.softmax_rows_ref(y), np.zeros((2, 3)))  # NaN rows -> 0


# ------------------------------------------------------------ attention ----

def test_attention_printed_seed42_weights():
    g = _golden("seed42_weights.json")
    q, k, v = tiny_example_qkv_f64()
    s = oracle.slopes_ref(4)
    out, w = oracle.attn_ref(q, k, v, s, causal=True, return_weights=True)
    assert list(out.shape) == g["shapes"]["output"]
    assert list(w.shape) == g["shapes"]["weights"]
    tol = 0.5 * 10.0 ** -g["decimals"] + 1e-9
    assert np.max(np.abs(w[0] - np.array(g["head_index_0"]))) <= tol
    assert np.max(np.abs(w[3] - np.array(g["head_index_3"]))) <= tol
    # and again from the fp32-rounded draw the device receives (rounding is far below 3 decimals)
    qf, kf, vf = tiny_example_qkv()
    _, w32 = oracle.attn_ref(qf, kf, vf, s, causal=True, return_weights=True)
    assert np.max(np.abs(w32[0] - np.array(g["head_index_0"]))) <= tol
    assert np.max(np.abs(w32[3] - np.array(g["head_index_3"]))) <= tol


def _equal_content_closed_form(m, n):
    w = np.zeros((n, n))
    r = math.exp(-m)
    for i in range(n):
        for j in range(i + 1):
            w[i, j] = r ** (i - j) * (1 - r) / (1 - r ** (i + 1))
    return w


@pytest.mark.parametrize("m", [0.5, 0.25, 0.0625, 2.0 ** -8])
def test_attention_equal_content_truncated_geometric(m):
    n, d = 12, 8
    q = np.zeros((1, n, d))
    rng = np.random.default_rng(1)
    k = rng.standard_normal((1, n, d))
    v = rng.standard_normal((1, n, d))
    out, w = oracle.attn_ref(q, k, v, [m], causal=True, return_weights=True)
    assert np.allclose(w[0], _equal_content_closed_form(m, n), rtol=1e-12, atol=1e-15)
    # each extra token of distance multiplies the weight by e^-m
    assert np.allclose(w[0, -1, :-1] / w[0, -1, 1:], math.exp(-m), rtol=1e-12)
    assert np.allclose(out[0], _equal_content_closed_form(m, n) @ v[0], rtol=1e-12, atol=1e-14)


def test_attention_rows_sum_to_one_and_mask_exact():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((2, 3, 33, 16)) for _ in range(3))
    _, w = oracle.attn_ref(q, k, v, oracle.slopes_ref(3), causal=True, return_weights=True)
    assert np.allclose(w.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert np.all(w[..., np.triu_indices(33, 1)[0], np.triu_indices(33, 1)[1]] == 0.0)


def _sdpa_bias_loops(n_q, n_k, m, causal, q_pos0=0):
    """Additive mask built element by element with loops (independent of the oracle)."""
    b = torch.zeros((n_q, n_k), dtype=torch.float64)
    for i in range(n_q):
        for j in range(n_k):
            pi = i + q_pos0
            if causal and j > pi:
                b[i, j] = float("-inf")
            else:
                b[i, j] = -m * abs(pi - j)
    return b


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_sdpa_with_explicit_bias(causal):
    rng = np.random.default_rng(3)
    B, H, N, d = 2, 6, 37, 24
    q, k, v = (rng.standard_normal((B, H, N, d)) for _ in range(3))
    s = oracle.slopes_ref(H)
    got = oracle.attn_ref(q, k, v, s, causal=causal)
    mask = torch.stack([_sdpa_bias_loops(N, N, float(s[h]), causal) for h in range(H)])[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), attn_mask=mask)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_zero_slope_is_causal_sdpa():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 4, 50, 32)) for _ in range(3))
    got = oracle.attn_ref(q, k, v, [0.0] * 4, causal=True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True)
    assert np.allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_key_position_form_equivalent():
    # row-shift invariance: -m(i-j) and +m j give the same softmax (abhik.ai and App. B.2)
    rng = np.random.default_rng(5)
    N, d, m = 29, 16, 0.3
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    _, w = oracle.attn_head_ref(q, k, v, m, causal=True)
    a = q @ k.T / math.sqrt(d) + m * np.arange(N)[None, :]
    a[np.triu_indices(N, 1)] = -np.inf
    assert np.allclose(w, scipy_softmax(a, axis=-1), rtol=1e-12, atol=1e-15)


def test_attention_prefix_invariance():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((1, 2, 40, 16)) for _ in range(3))
    s = oracle.slopes_ref(2)
    o1 = oracle.attn_ref(q, k, v, s)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    k2[..., 25:, :] = 30.0 * q[..., 25:, :]
    v2[..., 25:, :] = 1e4
    q2[..., 30:, :] = -7.0
    o2 = oracle.attn_ref(q2, k2, v2, s)
    assert np.array_equal(o1[..., :25, :], o2[..., :25, :])


def test_attention_bruteforce_tiny():
    q, k, v = tiny_example_qkv_f64()
    s = oracle.slopes_ref(4)
    for causal in (True, False):
        out, w = oracle.attn_ref(q, k, v, s, causal=causal, return_weights=True)
        bo, bw = oracle.attn_bruteforce(q, k, v, s, causal=causal)
        assert np.allclose(out, np.array(bo), rtol=1e-12, atol=1e-14)
        assert np.allclose(w, np.array(bw), rtol=1e-12, atol=1e-15)


@settings(max_examples=25, deadline=None)
@given(H=st.integers(1, 3), N=st.integers(1, 9), d=st.integers(1, 6),
       causal=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_attention_bruteforce_property(H, N, d, causal, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((H, N, d)) * 2 for _ in range(3))
    s = rng.uniform(0, 1, H)
    out = oracle.attn_ref(q, k, v, s, causal=causal)
    bo, _ = oracle.attn_bruteforce(q, k, v, s, causal=causal)
    assert np.allclose(out, np.array(bo), rtol=1e-11, atol=1e-12)


def test_rows_ref_matches_sdpa():
    rng = np.random.default_rng(7)
    N, d, m = 300, 32, 0.125
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    rows = [0, 1, 77, 150, 299]
    got = oracle.attn_rows_ref(q, k, v, m, rows, causal=True)
    mask = _sdpa_bias_loops(N, N, m, True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=mask[None])[0].numpy()
    assert np.allclose(got, ref[rows], rtol=1e-12, atol=1e-12)


def test_decode_matches_sdpa_single_query_and_last_forward_row():
    rng = np.random.default_rng(8)
    B, H, L, d = 2, 3, 70, 16
    kc, vc = (rng.standard_normal((B, H, L, d)) for _ in range(2))
    q = rng.standard_normal((B, H, d))
    s = oracle.slopes_ref(H)
    got = oracle.decode_ref(q, kc, vc, s)
    for b in range(B):
        for h in range(H):
            mask = _sdpa_bias_loops(1, L, float(s[h]), True, q_pos0=L - 1)
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, h])[None, None], torch.from_numpy(kc[b, h])[None],
                torch.from_numpy(vc[b, h])[None], attn_mask=mask[None])[0, 0].numpy()
            assert np.allclose(got[b, h], ref, rtol=1e-12, atol=1e-12)
    # the decode of the newest token equals the last row of the causal forward
    qf = rng.standard_normal((B, H, L, d))
    qf[:, :, -1, :] = q
    full = oracle.attn_ref(qf, kc, vc, s, causal=True)
    assert np.allclose(full[:, :, -1, :], got, rtol=1e-12, atol=1e-13)
    sub = oracle.decode_ref(q, kc, vc, s, pairs=[(1, 2), (0, 0)])
    assert np.array_equal(sub[0], got[1, 2]) and np.array_equal(sub[1], got[0, 0])
