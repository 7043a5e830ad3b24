"""Exact underflow skipping (ALIBI_SKIP_UNDERFLOW) on the GPU.

Skipping a key tile is allowed only where every weight it holds would round to
exactly zero ("When Attention Goes Blind", Sec. 3.2-3.3 underflow and the
wasted work of Sec. 5.1-5.2), so the output must be bit-identical to the same
call without skipping, which the other parity tests tie to the oracle. The
cases stress the bound: steep slopes, long rows, queries and keys with large
norms, position offsets, ragged lengths, d = 64 and 128.
"""
import numpy as np
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


def _pair(alibi, q, k, v, s, **kw):
    a = alibi.attn_fwd_ex(q, k, v, s, True, **kw)
    b = alibi.attn_fwd_ex(q, k, v, s, True, skip_underflow=True, **kw)
    torch.cuda.synchronize()
    return a, b


@pytest.mark.parametrize("B,H,N,d,recipe", [
    (2, 16, 4096, 128, None),       # the N = 4096, d = 128 shape, default slopes
    (1, 9, 2048, 64, "steep"),      # Sec. 4.2 steep slopes
    (1, 8, 3000, 128, "wide"),      # ragged length
    (2, 4, 1000, 64, None),
])
def test_skip_is_bit_exact(alibi, fwd_form, B, H, N, d, recipe):
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((B, H, N, d), seed=21))
    s = alibi.slopes(H) if recipe is None else alibi.slopes_recipe(recipe, H)
    a, b = _pair(alibi, q, k, v, s)
    assert torch.equal(a, b), f"max diff {(a.float() - b.float()).abs().max().item()}"


def test_skip_with_large_norms_is_bit_exact(alibi):
    # rows and keys with 8x the typical norm push the bound out and the true
    # maximum up; a few far keys aligned with a query test the bound itself
    B, H, N, d = 1, 4, 2048, 128
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=22)
    q[:, :, ::97] *= 8
    k[:, :, ::131] *= 8
    k[:, :, 5] = q[:, :, 1500] * 4          # key 5 strongly aligned with query 1500
    q, k, v = dev(q), dev(k), dev(v)
    s = alibi.slopes_recipe("steep", H)
    a, b = _pair(alibi, q, k, v, s)
    assert torch.equal(a, b)


def test_skip_with_offsets_is_bit_exact(alibi, fwd_form):
    q, _, _ = W.gaussian_qkv_bf16((1, 8, 300, 128), seed=23)
    _, k, v = W.gaussian_qkv_bf16((1, 8, 2000, 128), seed=24)
    q, k, v = dev(q), dev(k), dev(v)
    s = alibi.slopes(8)
    a, b = _pair(alibi, q, k, v, s, q_offset=1700)
    assert torch.equal(a, b)
    a, b = _pair(alibi, q, k, v, s, q_offset=2500, k_offset=100)   # queries after every key
    assert torch.equal(a, b)


def test_skip_flag_is_inert_elsewhere(alibi):
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((1, 4, 700, 64), seed=25))
    s = alibi.slopes(4)
    a, b = _pair(alibi, q, k, v, s, clamp=-87.0)
    assert torch.equal(a, b)
    z = torch.zeros(4, dtype=torch.float32)                        # zero slopes: nothing to skip
    a, b = _pair(alibi, q, k, v, z)
    assert torch.equal(a, b)


def test_skip_matches_oracle_sampled_rows(alibi):
    wl = W.FWD_B8_H16_N4096_D128
    q, k, v = W.gaussian_qkv_bf16((1, wl.H, wl.N, wl.d), seed=wl.seed)
    s = oracle.slopes_ref(wl.H)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), torch.from_numpy(s), True, skip_underflow=True)
    torch.cuda.synchronize()
    rows = np.array([0, 63, 64, 1000, 2047, 2048, 4000, wl.N - 1])
    for h in (0, 1, wl.H - 1):
        ref = oracle.attn_rows_ref(q[0, h], k[0, h], v[0, h], float(s[h]), rows)
        check_bf16(out[0, h, rows], ref, f"skip h={h}")


@pytest.mark.parametrize("B,H,N,d,recipe", [
    (2, 8, 2048, 128, "steep"),     # both sides skipped for most rows
    (1, 4, 3001, 64, "steep"),      # ragged length
    (1, 16, 4096, 128, None),       # default slopes
    (2, 3, 700, 128, "wide"),
])
def test_skip_non_causal_is_bit_exact(alibi, fwd_form, B, H, N, d, recipe):
    # without the mask the bias is -m |i - j|: tiles far on either side of a
    # block's queries hold only zero weights
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((B, H, N, d), seed=26))
    s = alibi.slopes(H) if recipe is None else alibi.slopes_recipe(recipe, H)
    a = alibi.attn_fwd_ex(q, k, v, s, False)
    b = alibi.attn_fwd_ex(q, k, v, s, False, skip_underflow=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b), f"max diff {(a.float() - b.float()).abs().max().item()}"


def test_skip_non_causal_with_offsets_is_bit_exact(alibi):
    q, _, _ = W.gaussian_qkv_bf16((1, 8, 300, 128), seed=27)
    _, k, v = W.gaussian_qkv_bf16((1, 8, 2000, 128), seed=28)
    q, k, v = dev(q), dev(k), dev(v)
    s = alibi.slopes_recipe("steep", 8)
    for qo, ko in ((1700, 0), (0, 900), (2500, 100)):
        a = alibi.attn_fwd_ex(q, k, v, s, False, q_offset=qo, k_offset=ko)
        b = alibi.attn_fwd_ex(q, k, v, s, False, q_offset=qo, k_offset=ko, skip_underflow=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b), (qo, ko)


def test_skip_non_causal_really_skips(alibi):
    # A NaN in V row j poisons every output row whose P against j is computed,
    # zero or not (0 NaN = NaN): the full forward poisons every row, the
    # skipping one only rows near j, on both sides.
    B, H, N, d = 1, 2, 2048, 128
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=29)
    v[:, :, 0, 0] = float("nan")        # far left of the last rows
    v[:, :, N - 1, 1] = float("nan")    # far right of the first rows
    q, k, v = dev(q), dev(k), dev(v)
    s = alibi.slopes_recipe("steep", H)
    a = alibi.attn_fwd_ex(q, k, v, s, False)
    b = alibi.attn_fwd_ex(q, k, v, s, False, skip_underflow=True)
    torch.cuda.synchronize()
    assert torch.isnan(a.float()).any(-1).all()
    nan_rows = torch.isnan(b.float()).any(-1)[0]       # (H, N)
    assert nan_rows[:, 0].all() and nan_rows[:, N - 1].all()  # the poisoned keys' own rows
    mid = nan_rows[:, N // 2 - 64: N // 2 + 64]
    print(f"[skip] non-causal: middle rows left finite: {int((~mid).sum())} of {mid.numel()}", flush=True)
    assert not mid.any()                                      # rows far from both keys skip both tiles
