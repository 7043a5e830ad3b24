"""Exact underflow skipping in the backward pass (needs an MI355X).

P = exp(logit - lse) is the only place the keys' distance enters the
gradients. Every logit of a (b, h) pair is at most A - m D with
A = max|q| max|k| / sqrt(d) (Cauchy-Schwarz), and every row's log-sum-exp is at
least its diagonal logit, so at least -A: pairs further apart than the
distance where 2 A - m D drops below the fp32 rounding limit have P that
rounds to exactly zero ("When Attention Goes Blind", Sec. 3.2-3.3), and with
it their dV and dS terms, hence their dK and dQ terms. The skipping backward
must therefore give the same bits as the full one, which the backward parity
tests tie to the fp64 oracle; one case here is also checked against the oracle
directly, and a planted NaN shows that the far tiles are really not visited.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import check_grads, dev

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


def _both(alibi, q, k, v, do, s, **kw):
    out, lse = alibi.attn_fwd_train(q, k, v, s, True) if not kw else (None, None)
    if out is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        out = alibi.attn_fwd_ex(q, k, v, s, True, lse=lse, **kw)
    a = alibi.attn_bwd(q, k, v, out, do, lse, s, True, **kw)
    b = alibi.attn_bwd(q, k, v, out, do, lse, s, True, skip_underflow=True, **kw)
    torch.cuda.synchronize()
    return a, b


def _same(a, b, tag):
    for x, y, n in zip(a, b, ("dq", "dk", "dv")):
        same = torch.equal(x, y)
        if not same:
            print(f"[parity] {tag} {n}: max diff {(x.float() - y.float()).abs().max().item():.3e}", flush=True)
        assert same, f"{tag} {n}"


# (B, H, N, d, slope recipe): the N = 4096 d = 128 shape at the default slopes
# (a third of the causal tiles skipped), steep slopes (most skipped), ragged
# lengths, a length below one key block, d = 64
CASES = [
    (1, 16, 4096, 128, None),
    (1, 9, 2048, 64, "steep"),
    (2, 4, 3001, 128, "steep"),
    (1, 8, 1000, 128, "wide"),
    (2, 3, 100, 64, "steep"),
]


@pytest.mark.parametrize("B,H,N,d,recipe", CASES)
def test_backward_skip_is_bit_exact(alibi, bwd_form, B, H, N, d, recipe):
    q, k, v, do = (dev(x) for x in _inputs((B, H, N, d), 41))
    s = alibi.slopes(H) if recipe is None else alibi.slopes_recipe(recipe, H)
    a, b = _both(alibi, q, k, v, do, s)
    _same(a, b, f"B{B} H{H} N{N} d{d} {recipe} qb={bwd_form}")


def test_backward_skip_with_large_norms_is_bit_exact(alibi):
    # rows with 8x the typical norm push the bound out and the true logits up;
    # a far key aligned with a query tests the bound itself
    q, k, v, do = _inputs((1, 4, 2048, 128), 42)
    q[:, :, ::97] *= 8
    k[:, :, ::131] *= 8
    k[:, :, 5] = q[:, :, 1500] * 4
    q, k, v, do = dev(q), dev(k), dev(v), dev(do)
    a, b = _both(alibi, q, k, v, do, alibi.slopes_recipe("steep", 4))
    _same(a, b, "large norms")


def test_backward_skip_matches_oracle(alibi):
    B, H, N, d = 1, 4, 1000, 64
    q, k, v, do = _inputs((B, H, N, d), 43)
    s = oracle.slopes_recipe_ref("steep", H, False)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    out, lse = alibi.attn_fwd_train(qd, kd, vd, torch.from_numpy(s), True)
    dq, dk, dv = alibi.attn_bwd(qd, kd, vd, out, dod, lse, torch.from_numpy(s), True, skip_underflow=True)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for h in range(H):
        check_grads((dq[0, h], dk[0, h], dv[0, h]), q[0, h], k[0, h], v[0, h], do[0, h], float(s[h]), True,
                    f"skip steep h={h}")


def test_backward_skip_really_skips(alibi):
    # A NaN in dO row i makes dS_ij = P_ij (dP_ij - D_i) NaN for every key
    # j <= i, zero P included, and dv_j NaN through P_ij dO_i: the full backward
    # spreads it to every key up to i, the skipping one only to keys it visits.
    B, H, N, d = 1, 2, 2048, 128
    q, k, v, do = _inputs((B, H, N, d), 44)
    i = N - 1
    do[:, :, i, 0] = float("nan")
    q, k, v, do = dev(q), dev(k), dev(v), dev(do)
    s = alibi.slopes_recipe("steep", H)
    out, lse = alibi.attn_fwd_train(q, k, v, s, True)
    _, dk_full, dv_full = alibi.attn_bwd(q, k, v, out, do, lse, s, True)
    dq, dk, dv = alibi.attn_bwd(q, k, v, out, do, lse, s, True, skip_underflow=True)
    torch.cuda.synchronize()
    for g in (dk_full, dv_full):
        assert torch.isnan(g[:, :, : i + 1].float()).any(-1).all()
    nan_keys = torch.isnan(dk.float()).any(-1)[0]          # (H, N)
    assert nan_keys[:, i].all()                              # the diagonal is always visited
    far = int((~nan_keys[:, : N // 2]).sum())
    print(f"[skip] keys of the first half left finite: {far} of {H * N // 2}", flush=True)
    assert far == H * N // 2                                 # steep slopes: the first half is never visited
    assert torch.equal(torch.isnan(dv.float()).any(-1)[0], nan_keys)
    # rows other than i are untouched by the NaN
    assert not torch.isnan(dq[:, :, :i].float()).any()


def test_backward_skip_flag_is_inert_elsewhere(alibi):
    q, k, v, do = (dev(x) for x in _inputs((1, 4, 700, 64), 45))
    s = alibi.slopes(4)
    a, b = _both(alibi, q, k, v, do, s, clamp=-87.0)
    _same(a, b, "clamp")
    a, b = _both(alibi, q, k, v, do, s, log_distance=True)
    _same(a, b, "log distance")
    a, b = _both(alibi, q, k, v, do, s, softcap=5.0)
    _same(a, b, "soft cap")
    out, lse = alibi.attn_fwd_train(q, k, v, s, False)
    a = alibi.attn_bwd(q, k, v, out, do, lse, s, False)
    b = alibi.attn_bwd(q, k, v, out, do, lse, s, False, skip_underflow=True)
    _same(a, b, "non-causal")
    z = torch.zeros(4, dtype=torch.float32)                  # zero slopes: nothing to skip
    a, b = _both(alibi, q, k, v, do, z)
    _same(a, b, "zero slopes")


@pytest.mark.parametrize("B,H,N,d,recipe", [
    (1, 8, 2048, 128, "steep"),
    (2, 3, 1000, 64, "steep"),
    (1, 16, 4096, 128, None),
])
def test_backward_skip_non_causal_is_bit_exact(alibi, bwd_form, B, H, N, d, recipe):
    # the symmetric bias -m |i - j|: tiles far on either side carry zero P
    q, k, v, do = (dev(x) for x in _inputs((B, H, N, d), 46))
    s = alibi.slopes(H) if recipe is None else alibi.slopes_recipe(recipe, H)
    out, lse = alibi.attn_fwd_train(q, k, v, s, False)
    a = alibi.attn_bwd(q, k, v, out, do, lse, s, False)
    b = alibi.attn_bwd(q, k, v, out, do, lse, s, False, skip_underflow=True)
    torch.cuda.synchronize()
    _same(a, b, f"non-causal B{B} H{H} N{N} d{d} {recipe} qb={bwd_form}")


def test_backward_skip_non_causal_really_skips(alibi):
    # NaN in dO of the middle row: the full backward spreads it to every key,
    # the skipping one only to keys near that row, on both sides
    B, H, N, d = 1, 2, 2048, 128
    q, k, v, do = _inputs((B, H, N, d), 47)
    i = N // 2
    do[:, :, i, 0] = float("nan")
    q, k, v, do = dev(q), dev(k), dev(v), dev(do)
    s = alibi.slopes_recipe("steep", H)
    out, lse = alibi.attn_fwd_train(q, k, v, s, False)
    _, dk_full, _ = alibi.attn_bwd(q, k, v, out, do, lse, s, False)
    dq, dk, dv = alibi.attn_bwd(q, k, v, out, do, lse, s, False, skip_underflow=True)
    torch.cuda.synchronize()
    assert torch.isnan(dk_full.float()).any(-1).all()
    nan_keys = torch.isnan(dk.float()).any(-1)[0]           # (H, N)
    assert nan_keys[:, i].all()
    print(f"[skip] non-causal keys left finite: {int((~nan_keys).sum())} of {H * N}", flush=True)
    assert not nan_keys[:, :64].any() and not nan_keys[:, -64:].any()   # both ends are never visited
    assert torch.equal(torch.isnan(dv.float()).any(-1)[0], nan_keys)
