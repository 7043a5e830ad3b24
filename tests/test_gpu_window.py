"""GPU parity of the hard per-head window against the oracle.

"When Attention Goes Blind", Sec. 5.2 (steep heads act as sliding windows) and
Sec. 5.3 (a hard window lets the computation skip out-of-window entries): a
window of W tokens keeps key c for query r when 0 <= pos(r) - pos(c) < W
(oracle.variant_head_ref, window=W). The bf16 MFMA forward (in its 4-wave,
8-wave and key-range-split forms), the generic kernels (fp32 and bf16 of other
head sizes), offsets, the log-sum-exp output and the exact skipping are
compared with the oracle or, where the windowed result must not change, bit for
bit with the call without the window.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Bf16Stats, F32_TOL, LSE_TOL, check_bf16, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


def _case(alibi, shape_q, shape_kv, s, wins, qo=0, ko=0, seed=51, **kw):
    q, _, _ = W.gaussian_qkv_bf16(shape_q, seed=seed)
    _, k, v = W.gaussian_qkv_bf16(shape_kv, seed=seed + 1)
    ref = oracle.variant_ref(q, k, v, s, True, q_offset=qo, k_offset=ko, windows=wins)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), torch.as_tensor(s), True, q_offset=qo, k_offset=ko,
                            window=wins, **kw)
    torch.cuda.synchronize()
    return out, ref, (q, k, v)


@pytest.mark.parametrize("B,H,N,d", [(1, 8, 300, 128), (2, 8, 777, 64), (1, 8, 1030, 128), (2, 6, 129, 64)])
def test_window_bf16(alibi, fwd_form, B, H, N, d):
    # windows inside a tile, at and around tile edges (64 keys), across blocks, beyond N
    wins = [1, 2, 63, 64, 65, 200, 513, N + 7][:H]
    s = oracle.slopes_ref(H)
    out, ref, _ = _case(alibi, (B, H, N, d), (B, H, N, d), s, wins)
    check_bf16(out, ref, f"window B{B} H{H} N{N} d{d} {fwd_form}")


@pytest.mark.parametrize("Nq,Nk,qo", [(100, 300, 200), (77, 1500, 1423), (300, 300, 0)])
def test_window_bf16_chunked_prefill(alibi, fwd_form, Nq, Nk, qo):
    s = oracle.slopes_ref(4)
    wins = [5, 100, 333, 4000]
    out, ref, _ = _case(alibi, (2, 4, Nq, 128), (2, 4, Nk, 128), s, wins, qo=qo)
    check_bf16(out, ref, f"window chunk {Nq},{Nk},{qo} {fwd_form}")


def test_window_one_token_is_the_own_value_row(alibi):
    q, k, v = W.gaussian_qkv_bf16((1, 4, 200, 128), seed=53)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), alibi.slopes(4), True, window=[1, 1, 1, 1])
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), v)


def test_window_zero_gives_zero_rows(alibi):
    q, k, v = W.gaussian_qkv_bf16((1, 2, 150, 64), seed=54)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), alibi.slopes(2), True, window=[0, -5])
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


@pytest.mark.parametrize("d", [64, 128])
def test_window_covering_every_key_is_bitwise_the_plain_call(alibi, d):
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((2, 4, 700, d), seed=55))
    s = alibi.slopes(4)
    lse0 = torch.empty((2, 4, 700), dtype=torch.float32, device="cuda")
    lse1 = torch.empty_like(lse0)
    a = alibi.attn_fwd_ex(q, k, v, s, True, lse=lse0)
    b = alibi.attn_fwd_ex(q, k, v, s, True, lse=lse1, window=[700, 701, 10 ** 6, 2 ** 31 - 1])
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(lse0, lse1)


def test_window_with_skipping_is_bitwise_the_window_alone(alibi, fwd_form):
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((1, 8, 2048, 128), seed=56))
    s = alibi.slopes_recipe("steep", 8)
    wins = [16, 100, 300, 600, 1000, 1500, 2000, 4096]
    a = alibi.attn_fwd_ex(q, k, v, s, True, window=wins)
    b = alibi.attn_fwd_ex(q, k, v, s, True, window=wins, skip_underflow=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_window_lse_one_token_is_the_diagonal_logit(alibi):
    # with a one-token window the row's log-sum-exp is its own logit q.k / sqrt(d)
    q, k, v = W.gaussian_qkv_bf16((1, 3, 333, 128), seed=57)
    lse = torch.empty((1, 3, 333), dtype=torch.float32, device="cuda")
    alibi.attn_fwd_ex(dev(q), dev(k), dev(v), alibi.slopes(3), True, lse=lse, window=[1, 1, 1])
    torch.cuda.synchronize()
    qd, kd = q.double().numpy(), k.double().numpy()
    ref = np.einsum("bhnd,bhnd->bhn", qd, kd) / np.sqrt(128.0)
    assert np.abs(lse.cpu().double().numpy() - ref).max() <= LSE_TOL


@pytest.mark.parametrize("d", [16, 96])
def test_window_generic_kernels(alibi, d):
    s = oracle.slopes_ref(3)
    wins = [1, 9, 40]
    q, k, v = W.gaussian_qkv_f32((2, 3, 57, d), seed=58)
    ref = oracle.variant_ref(q, k, v, s, True, q_offset=4, windows=wins)
    out = alibi.attn_fwd_ex(*(dev(torch.from_numpy(x)) for x in (q, k, v)), torch.from_numpy(s), True,
                            q_offset=4, window=wins)
    torch.cuda.synchronize()
    err = np.abs(out.cpu().double().numpy() - ref).max()
    print(f"[parity] fp32 window d{d}: {err:.2e}", flush=True)
    assert err <= F32_TOL
    if d % 8 == 0:
        qb, kb, vb = W.gaussian_qkv_bf16((1, 3, 57, d), seed=59)
        ref = oracle.variant_ref(qb, kb, vb, s, True, windows=wins)
        out = alibi.attn_fwd_ex(dev(qb), dev(kb), dev(vb), torch.from_numpy(s), True, window=wins)
        check_bf16(out, ref, f"bf16 generic window d{d}")


def test_window_full_size_every_element(alibi):
    # the N = 4096, d = 128 shape, one batch of 16 heads, each with the window
    # its slope reaches the fp32 denormal limit at (124 tokens for the steepest)
    wl = W.FWD_B8_H16_N4096_D128
    q, k, v = W.gaussian_qkv_bf16((1, wl.H, wl.N, wl.d), seed=wl.seed + 2)
    s = oracle.slopes_ref(wl.H)
    wins = [int(np.ceil(oracle.TAU_D / float(m))) for m in s]
    assert wins[0] == 124
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), torch.from_numpy(s), True, window=wins).cpu()
    st = Bf16Stats("N4096 d128 blindness windows")
    for h in range(wl.H):
        ref = oracle.variant_head_ref(q[0, h], k[0, h], v[0, h], s[h], True, window=wins[h])[0]
        st.add(out[0, h], ref)
    st.finish()
