"""Pins of the oracle's mitigation variants and slope recipes (CPU only).

Printed values: App. F Table 8 and Sec. 4.2 / 4.3 of "When Attention Goes
Blind: Numerical Failure in ALiBi Positional Encodings", stored in
tests/golden/slope_recipes_table8.json. The rest are closed forms the
definitions of Sec. 3.4 fix by hand (harmonic weights for log distances, the
saturation of tanh, a floor that flattens every distant key), limits that
reduce a variant to plain ALiBi or to PyTorch's causal SDPA, and the
row-selection property of query/key position offsets.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _g():
    with open(os.path.join(GOLDEN, "slope_recipes_table8.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("recipe", ["steep", "safe", "wide", "explicit"])
def test_recipes_reproduce_table8(recipe):
    g = _g()
    m = oracle.slopes_recipe_ref(recipe, g["H"])
    assert m.dtype == np.float32
    # the threshold as Table 4 prints it (4 decimals), not the oracle's constant
    with open(os.path.join(GOLDEN, "underflow_tables.json")) as f:
        tau = -json.load(f)["table4"]["fp32"]["tau_d"]
    got = [int(round(tau / float(x))) for x in m]
    assert got == g["table8"][recipe]


def test_threshold_constant_is_the_fp32_normal_limit():
    assert abs(oracle.TAU_D + oracle.format_thresholds("fp32")["tau_d"]) < 1e-12


@pytest.mark.parametrize("recipe", ["steep", "safe", "wide"])
def test_recipe_endpoints_sec42(recipe):
    lo, hi = _g()["sec42_endpoints"][recipe]
    for H in (2, 9, 16, 32):
        d = oracle.recipe_distances(recipe, H)
        assert d[0] == lo and abs(d[-1] - hi) < 1e-9 * hi
        assert np.all(np.diff(d) > 0)          # steepest head first
        r = d[1:] / d[:-1]
        assert np.allclose(r, r[0], rtol=1e-12)  # geometric spacing


def test_explicit_doubles_from_32():
    d = oracle.recipe_distances("explicit", 12)
    assert d[0] == 32 and np.all(d[1:] == 2 * d[:-1])


def test_log_adapted_slopes_keep_the_target_distance():
    # Sec. 4.3: with log distances the explicit slopes become |tau| / log(delta + 1),
    # so the log-scaled blindness distance (pinned to Sec. 3.4's 4.37e53 elsewhere)
    # lands back on the target
    for recipe in ("explicit", "wide", "safe"):
        dl = oracle.recipe_distances(recipe, 9)
        m = oracle.slopes_recipe_ref(recipe, 9, log_distance=True)
        for t, s in zip(dl, m):
            got = oracle.log_scaled_blindness_distance(float(s), -oracle.TAU_D)
            assert abs(got - t) <= 2e-5 * t * math.log(t + 1) + 1e-6


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_no_mitigation_equals_plain_alibi():
    q, k, v = _rand((10, 8), 1), _rand((10, 8), 2), _rand((10, 8), 3)
    for causal in (True, False):
        o1, w1 = oracle.variant_head_ref(q, k, v, 0.3, causal)
        o2, w2 = oracle.attn_head_ref(q, k, v, 0.3, causal)
        assert np.allclose(o1, o2, atol=1e-14) and np.allclose(w1, w2, atol=1e-14)


def test_limits_reduce_to_plain_alibi():
    q, k, v = _rand((12, 8), 4), _rand((12, 8), 5), _rand((12, 8), 6)
    o_plain, _ = oracle.attn_head_ref(q, k, v, 0.5, True)
    o_c, _ = oracle.variant_head_ref(q, k, v, 0.5, True, clamp=-1e30)   # floor never reached
    o_s, _ = oracle.variant_head_ref(q, k, v, 0.5, True, softcap=1e9)   # tanh(x) = x
    assert np.allclose(o_c, o_plain, atol=1e-14)
    assert np.allclose(o_s, o_plain, atol=1e-9)


def test_clamp_at_zero_is_causal_sdpa():
    import torch
    q, k, v = _rand((2, 3, 9, 8), 7), _rand((2, 3, 9, 8), 8), _rand((2, 3, 9, 8), 9)
    got = oracle.variant_ref(q, k, v, [0.5, 0.25, 2.0], causal=True, clamp=0.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True).numpy()
    assert np.allclose(got, ref, atol=1e-12)


def test_clamp_closed_form_flattens_distant_keys():
    # A = 0 and a slope so steep that every key but the query itself sits on the
    # floor: row i puts 1 / (1 + i e^c) on itself and e^c / (1 + i e^c) elsewhere
    c = -87.0
    n = 6
    z = np.zeros((n, 4))
    _, w = oracle.variant_head_ref(z, z, z, 100.0, True, clamp=c)
    for i in range(n):
        den = 1.0 + i * math.exp(c)
        assert abs(w[i, i] - 1.0 / den) < 1e-15
        for j in range(i):
            assert abs(w[i, j] - math.exp(c) / den) / (math.exp(c) / den) < 1e-12


def test_log_distance_harmonic_weights():
    # A = 0, slope 1, log distances: weight (i - j + 1)^-1 / H_{i+1} (harmonic number)
    z = np.zeros((5, 4))
    _, w = oracle.variant_head_ref(z, z, z, 1.0, True, log_distance=True)
    assert np.allclose(w[3, :4], [0.12, 0.16, 0.24, 0.48], atol=1e-15)   # H_4 = 25/12
    assert np.allclose(w[1, :2], [1 / 3, 2 / 3], atol=1e-15)
    # slope 2: (D + 1)^-2 over sum_t (t + 1)^-2
    _, w2 = oracle.variant_head_ref(z, z, z, 2.0, True, log_distance=True)
    den = 1 + 1 / 4 + 1 / 9
    assert np.allclose(w2[2, :3], [(1 / 9) / den, (1 / 4) / den, 1 / den], atol=1e-15)


def test_log_distance_symmetric_without_mask():
    z = np.zeros((5, 4))
    _, w = oracle.variant_head_ref(z, z, z, 1.0, False, log_distance=True)
    row = np.array([1 / 3, 1 / 2, 1.0, 1 / 2, 1 / 3])      # row 2: |D| = 2, 1, 0, 1, 2
    assert np.allclose(w[2], row / row.sum(), atol=1e-15)


def test_softcap_saturates_at_z():
    # slope 0, two keys: A_0 far above z, A_1 = 0 -> logits z and 0 -> weights e^z / (1 + e^z)
    d = 4
    q = np.zeros((2, d)); q[1, 0] = 1.0
    k = np.zeros((2, d)); k[0, 0] = 1e6 * math.sqrt(d)
    v = np.eye(2, d)
    for z in (1.0, 3.0):
        _, w = oracle.variant_head_ref(q, k, v, 0.0, True, softcap=z)
        assert abs(w[1, 0] - math.exp(z) / (1 + math.exp(z))) < 1e-15
        assert abs(w[1, 1] - 1 / (1 + math.exp(z))) < 1e-15


def test_softcap_caps_content_not_bias():
    # content zero: the cap changes nothing, the bias still acts in full
    z = np.zeros((7, 4))
    _, w = oracle.variant_head_ref(z, z, z, 3.0, True, softcap=0.5)
    _, w_plain = oracle.attn_head_ref(z, z, z, 3.0, True)
    assert np.allclose(w, w_plain, atol=1e-15)


def test_offsets_select_rows_of_the_full_forward():
    # a chunk of queries at positions s.. against all keys from 0 is the tail of the
    # full causal forward (chunked prefill); shifting both offsets changes nothing
    q, k, v = _rand((1, 2, 20, 8), 10), _rand((1, 2, 20, 8), 11), _rand((1, 2, 20, 8), 12)
    sl = [0.5, 0.125]
    full = oracle.attn_ref(q, k, v, sl, causal=True)
    for s in (1, 7, 19):
        part = oracle.variant_ref(q[:, :, s:], k, v, sl, True, q_offset=s)
        assert np.allclose(part, full[:, :, s:], atol=1e-13)
        moved = oracle.variant_ref(q[:, :, s:], k, v, sl, True, q_offset=s + 1000, k_offset=1000)
        assert np.allclose(moved, part, atol=1e-13)
    full_nc = oracle.attn_ref(q, k, v, sl, causal=False)
    part_nc = oracle.variant_ref(q[:, :, 5:], k, v, sl, False, q_offset=5)
    assert np.allclose(part_nc, full_nc[:, :, 5:], atol=1e-13)


def test_rows_without_visible_keys_are_zero():
    q, k, v = _rand((1, 1, 4, 8), 13), _rand((1, 1, 6, 8), 14), _rand((1, 1, 6, 8), 15)
    out = oracle.variant_ref(q, k, v, [0.5], True, q_offset=0, k_offset=2)
    assert np.all(out[0, 0, :2] == 0.0)       # positions 0, 1 see no key (keys start at 2)
    assert np.all(np.isfinite(out)) and np.any(out[0, 0, 2:] != 0.0)
