"""GPU parity of the extended forward (mitigations, position offsets) against the oracle.

Sec. 3.4 mitigations of "When Attention Goes Blind" (bias floor, ln(D + 1)
distances, soft-capped content logits), every combination, with and without
the causal mask, and query/key position offsets (chunked prefill, rows that
see no key). Calls go through the C ABI; the oracle (oracle.variant_ref) sees
the same fp32 or bf16 values. Tolerances as in tests/parity_util.py.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import Bf16Stats, F32_TOL, check_bf16, dev

pytestmark = pytest.mark.gpu

FLAGS = list(itertools.product([None, -3.0], [False, True], [None, 2.0]))  # clamp, log, softcap


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


def _ids(f):
    c, l, s = f
    return f"c{int(c is not None)}l{int(l)}s{int(s is not None)}"


# ------------------------------------------------------------ fp32 generic --

@pytest.mark.parametrize("flags", FLAGS, ids=_ids)
@pytest.mark.parametrize("causal", [True, False])
def test_fp32_variants(alibi, flags, causal):
    clamp, logd, cap = flags
    q, k, v = W.gaussian_qkv_f32((1, 3, 37, 16), seed=3)
    s = oracle.slopes_ref(3)
    ref = oracle.variant_ref(q, k, v, s, causal, clamp, logd, cap)
    out = alibi.attn_fwd_ex(dev(torch.from_numpy(q)), dev(torch.from_numpy(k)), dev(torch.from_numpy(v)),
                            torch.from_numpy(s), causal, clamp=clamp, log_distance=logd, softcap=cap)
    err = np.abs(out.cpu().double().numpy() - ref).max()
    print(f"[parity] fp32 variant {_ids(flags)} causal={causal}: max err {err:.2e}", flush=True)
    assert err <= F32_TOL


@pytest.mark.parametrize("Nq,Nk,qo,ko,causal", [
    (11, 40, 29, 0, True),     # chunked prefill: the last 11 of 40 tokens
    (9, 20, 3, 10, True),      # rows 0..6 see no key -> zero rows
    (12, 30, 5, 2, False),     # symmetric bias with shifted positions
    (16, 16, 1000, 1000, True),  # both offsets shifted: no change
])
def test_fp32_offsets(alibi, Nq, Nk, qo, ko, causal):
    q, _, _ = W.gaussian_qkv_f32((2, 2, Nq, 24), seed=5)
    _, k, v = W.gaussian_qkv_f32((2, 2, Nk, 24), seed=6)
    s = np.array([0.5, 0.0625], dtype=np.float32)
    ref = oracle.variant_ref(q, k, v, s, causal, q_offset=qo, k_offset=ko)
    out = alibi.attn_fwd_ex(dev(torch.from_numpy(q)), dev(torch.from_numpy(k)), dev(torch.from_numpy(v)),
                            torch.from_numpy(s), causal, q_offset=qo, k_offset=ko)
    got = out.cpu().double().numpy()
    err = np.abs(got - ref).max()
    print(f"[parity] fp32 offsets {Nq},{Nk},{qo},{ko},{causal}: max err {err:.2e}", flush=True)
    assert err <= F32_TOL
    dead = ref.reshape(-1, 24)
    assert np.all(got.reshape(-1, 24)[np.all(dead == 0.0, axis=1)] == 0.0)


# ------------------------------------------------------------ bf16 MFMA -----

def _bf16_case(alibi, shape_q, shape_kv, slopes, causal, clamp, logd, cap, qo=0, ko=0, seed=7):
    q, _, _ = W.gaussian_qkv_bf16(shape_q, seed=seed)
    _, k, v = W.gaussian_qkv_bf16(shape_kv, seed=seed + 1)
    ref = oracle.variant_ref(q, k, v, slopes, causal, clamp, logd, cap, qo, ko)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), torch.as_tensor(slopes), causal, clamp=clamp,
                            log_distance=logd, softcap=cap, q_offset=qo, k_offset=ko)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("flags", FLAGS, ids=_ids)
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
def test_bf16_mfma_variants(alibi, fwd_waves, flags, d, causal):
    clamp, logd, cap = flags
    cap = None if cap is None else 5.0
    clamp = None if clamp is None else -10.0
    s = oracle.slopes_ref(4)
    out, ref = _bf16_case(alibi, (1, 4, 300, d), (1, 4, 300, d), s, causal, clamp, logd, cap)
    check_bf16(out, ref, f"mfma variant {_ids(flags)} d={d} causal={causal}")


@pytest.mark.parametrize("recipe", ["steep", "safe", "wide", "explicit"])
def test_bf16_paper_settings_with_recipes(alibi, recipe):
    # Sec. 4.3: c_clamp = -87, z = 50, recipe slopes (log-adapted when log-scaled)
    H, N = 9, 700
    for logd in (False, True):
        s = oracle.slopes_recipe_ref(recipe, H, logd)
        assert np.array_equal(alibi.slopes_recipe(recipe, H, logd).numpy(), s)
        out, ref = _bf16_case(alibi, (1, H, N, 128), (1, H, N, 128), s, True, -87.0, logd, 50.0, seed=11)
        check_bf16(out, ref, f"paper settings {recipe} log={logd}")


@pytest.mark.parametrize("Nq,Nk,qo,ko,causal", [
    (100, 300, 200, 0, True),    # chunked prefill across several key tiles
    (77, 333, 256, 0, True),     # ragged chunk and ragged cache
    (200, 150, 0, 100, True),    # the first 100 query rows see no key
    (130, 90, 500, 0, True),     # every query after every key
    (150, 260, 40, 0, False),    # symmetric bias, shifted queries
    (64, 64, 4096, 4096, True),  # both offsets shifted
])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_mfma_offsets(alibi, fwd_form, Nq, Nk, qo, ko, causal, d):
    s = oracle.slopes_ref(2)
    out, ref = _bf16_case(alibi, (2, 2, Nq, d), (2, 2, Nk, d), s, causal, None, False, None, qo, ko)
    check_bf16(out, ref, f"mfma offsets {Nq},{Nk},{qo},{ko},{causal} d={d}")
    got = out.cpu().double().numpy()
    zero_rows = np.all(ref == 0.0, axis=-1)
    assert np.all(got[zero_rows] == 0.0)


def test_bf16_offsets_with_all_mitigations(alibi, fwd_waves):
    s = oracle.slopes_recipe_ref("wide", 3)
    out, ref = _bf16_case(alibi, (1, 3, 90, 128), (1, 3, 400, 128), s, True, -20.0, True, 8.0, 310, 0)
    check_bf16(out, ref, "mfma chunk + all mitigations")


def test_bf16_generic_head_size_variants(alibi):
    s = oracle.slopes_ref(3)
    out, ref = _bf16_case(alibi, (1, 3, 70, 96), (1, 3, 90, 96), s, True, -4.0, True, 3.0, 20, 0)
    check_bf16(out, ref, "generic d=96 all mitigations + offsets")


def test_plain_ex_matches_plain_forward_bitwise(alibi):
    # no mitigation and no offsets: the same kernel as alibi_attn_fwd
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((2, 4, 333, 128), seed=13))
    s = alibi.slopes(4)
    a = alibi.attn_fwd(q, k, v, s, causal=True)
    b = alibi.attn_fwd_ex(q, k, v, s, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bf16_all_mitigations_full_size_every_element(alibi):
    # the N = 4096, d = 128 shape with every mitigation at the paper's settings;
    # every element of two batches (32 heads) against the oracle, head by head
    wl = W.FWD_B8_H16_N4096_D128
    shape = (2, wl.H, wl.N, wl.d)
    q, k, v = W.gaussian_qkv_bf16(shape, seed=wl.seed)
    s = oracle.slopes_recipe_ref("steep", wl.H, log_distance=True)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), torch.from_numpy(s), True,
                            clamp=-87.0, log_distance=True, softcap=50.0).cpu()
    st = Bf16Stats("N4096 d128 clamp + log distance + soft cap")
    for b in range(shape[0]):
        for h in range(wl.H):
            ref = oracle.variant_head_ref(q[b, h], k[b, h], v[b, h], s[h], True, -87.0, True, 50.0)[0]
            st.add(out[b, h], ref)
    st.finish()


def test_bf16_clamp_full_size_every_element(alibi):
    # the bias floor alone at the paper's c_clamp = -87 on the N = 4096, d = 128
    # shape: with the standard slopes some heads reach the floor within a few
    # hundred keys and some never do, so open tiles of all three kinds (wholly
    # above the floor, wholly on it, crossing it) occur; every element of 16 heads
    wl = W.FWD_B8_H16_N4096_D128
    shape = (1, wl.H, wl.N, wl.d)
    q, k, v = W.gaussian_qkv_bf16(shape, seed=wl.seed + 1)
    s = oracle.slopes_ref(wl.H)
    out = alibi.attn_fwd_ex(dev(q), dev(k), dev(v), torch.from_numpy(s), True, clamp=-87.0).cpu()
    st = Bf16Stats("N4096 d128 clamp -87")
    for h in range(wl.H):
        ref = oracle.variant_head_ref(q[0, h], k[0, h], v[0, h], s[h], True, -87.0)[0]
        st.add(out[0, h], ref)
    st.finish()


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_clamp_signed_slopes(alibi, fwd_waves, d):
    # slopes of either sign (a negative slope raises the bias with distance, so
    # the floor binds near the diagonal instead of far from it) and zero
    s = np.array([-0.05, 0.3, -0.001, 0.0, 0.02, 1.5], dtype=np.float32)
    out, ref = _bf16_case(alibi, (1, 6, 700, d), (1, 6, 700, d), s, True, -6.0, False, None, seed=17)
    check_bf16(out, ref, f"clamp signed slopes d={d}")
