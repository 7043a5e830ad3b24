"""GPU parity of the HIP path against the fp64 oracle (needs an MI355X).

Every call goes through the C ABI (the ctypes binding); the oracle sees the
same fp32 or bf16 values the device sees, upcast exactly.

Tolerances (tests/parity_util.py):
* fp32 path: max |gpu - oracle| <= 1e-5 on outputs and weights.
* bf16 paths: every element satisfies |gpu - o| <= 1e-2 + ulp_bf16(o) / 2.
* masking: masked weights are exactly 0 and rows before a changed future are
  bitwise unchanged; slopes are bitwise.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W

from parity_util import BF16_TOL, F32_TOL, check_bf16, dev, half_ulp_bf16  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()  # raises if the HIP library is missing: no fallback
    return mod


# ------------------------------------------------------------- fp32 path ----

def test_tiny_fp32_outputs_and_weights(alibi):
    q, k, v = W.tiny_example_qkv()
    s = oracle.slopes_ref(4)
    ref_o, ref_w = oracle.attn_ref(q, k, v, s, causal=True, return_weights=True)
    qd, kd, vd = (dev(torch.from_numpy(x)[None]) for x in (q, k, v))
    sd = alibi.slopes(4)
    assert np.array_equal(sd.numpy(), s)
    out = alibi.attn_fwd_f32(qd, kd, vd, sd, causal=True)
    w = alibi.attn_weights_f32(qd, kd, sd, causal=True)
    torch.cuda.synchronize()
    eo = np.abs(out[0].cpu().double().numpy() - ref_o).max()
    ew = np.abs(w[0].cpu().double().numpy() - ref_w).max()
    print(f"[parity] tiny fp32: out err {eo:.2e}, weights err {ew:.2e}", flush=True)
    assert eo <= F32_TOL and ew <= F32_TOL
    wn = w[0].cpu().numpy()
    iu = np.triu_indices(8, 1)
    assert np.all(wn[:, iu[0], iu[1]] == 0.0)  # masked weights exactly zero
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "seed42_weights.json")))
    assert np.abs(wn[0] - np.array(g["head_index_0"])).max() <= 5e-4 + 1e-6
    assert np.abs(wn[3] - np.array(g["head_index_3"])).max() <= 5e-4 + 1e-6


@pytest.mark.parametrize("B,H,N,d,causal", [(2, 3, 37, 16, True), (1, 6, 130, 33, True),
                                             (1, 2, 65, 256, True), (2, 5, 50, 7, False),
                                             (1, 1, 1, 16, True)])
def test_fp32_generic_shapes(alibi, B, H, N, d, causal):
    q, k, v = W.gaussian_qkv_f32((B, H, N, d), seed=B * 1000 + N)
    s = oracle.slopes_ref(H)
    ref = oracle.attn_ref(q, k, v, s, causal=causal)
    out = alibi.attn_fwd_f32(*(dev(torch.from_numpy(x)) for x in (q, k, v)), alibi.slopes(H), causal=causal)
    err = np.abs(out.cpu().double().numpy() - ref).max()
    print(f"[parity] fp32 B{B} H{H} N{N} d{d} causal={causal}: {err:.2e}", flush=True)
    assert err <= F32_TOL


# ------------------------------------------------------- bf16 forward path ----

FWD_SMALL = [
    (1, 1, 1, 64, True), (1, 2, 7, 128, True), (2, 3, 63, 64, True), (1, 4, 64, 128, True),
    (1, 4, 65, 128, True), (2, 6, 129, 64, True), (1, 9, 200, 128, True), (1, 12, 300, 64, True),
    (2, 20, 257, 128, True), (1, 3, 513, 128, True), (1, 71, 40, 64, True),
    (1, 2, 1, 128, False), (1, 3, 100, 64, False), (2, 4, 190, 128, False), (1, 2, 600, 128, False),
]


@pytest.mark.parametrize("B,H,N,d,causal", FWD_SMALL)
def test_fwd_bf16_small(alibi, fwd_form, B, H, N, d, causal):
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=7 + N + H)
    s = oracle.slopes_ref(H)
    ref = oracle.attn_ref(q, k, v, s, causal=causal)
    out = alibi.attn_fwd(dev(q), dev(k), dev(v), alibi.slopes(H), causal=causal)
    check_bf16(out, ref, f"fwd B{B} H{H} N{N} d{d} causal={causal}")


@pytest.mark.parametrize("d", [32, 96, 256])
def test_fwd_bf16_generic_head_sizes(alibi, d):
    B, H, N = 1, 3, 77
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=d)
    ref = oracle.attn_ref(q, k, v, oracle.slopes_ref(H), causal=True)
    out = alibi.attn_fwd(dev(q), dev(k), dev(v), alibi.slopes(H), causal=True)
    check_bf16(out, ref, f"fwd generic d{d}")


@pytest.mark.parametrize("wl", [W.FWD_B8_H8_N1024_D64, W.FWD_B4_H12_N2048_D64], ids=lambda w: w.name)
def test_fwd_bf16_full_configs_every_element(alibi, wl):
    q, k, v = W.gaussian_qkv_bf16(wl.shape, seed=wl.seed)
    ref = oracle.attn_ref(q, k, v, oracle.slopes_ref(wl.H), causal=True)
    out = alibi.attn_fwd(dev(q), dev(k), dev(v), alibi.slopes(wl.H), causal=True)
    check_bf16(out, ref, wl.name)


def test_fwd_causality_poison_bitwise(alibi, fwd_form):
    B, H, N, d = 1, 4, 300, 128
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=11)
    s = alibi.slopes(H)
    o1 = alibi.attn_fwd(dev(q), dev(k), dev(v), s, causal=True)
    cut = 150
    k2, v2 = k.clone(), v.clone()
    k2[:, :, cut:] = (30.0 * q[:, :, cut:].float()).to(torch.bfloat16)
    v2[:, :, cut:] = 1e4
    o2 = alibi.attn_fwd(dev(q), dev(k2), dev(v2), s, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1[:, :, :cut], o2[:, :, :cut])
    assert torch.isfinite(o2.float()).all()


def test_fwd_deterministic(alibi):
    q, k, v = (dev(x) for x in W.gaussian_qkv_bf16((2, 8, 700, 128), seed=3))
    s = alibi.slopes(8)
    a = alibi.attn_fwd(q, k, v, s)
    b = alibi.attn_fwd(q, k, v, s)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_fwd_zero_slopes_match_sdpa(alibi):
    # m = 0 reduces to plain causal attention; compare against the oracle and
    # also sanity-check against torch's fp32 SDPA on the CPU
    B, H, N, d = 1, 4, 257, 64
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=5)
    zero = torch.zeros(H, dtype=torch.float32)
    out = alibi.attn_fwd(dev(q), dev(k), dev(v), zero, causal=True)
    ref = oracle.attn_ref(q, k, v, np.zeros(H), causal=True)
    check_bf16(out, ref, "fwd zero slopes")


# --------------------------------------------------------------- decode ----

DEC_SMALL = [(1, 1, 1, 128), (1, 2, 7, 64), (2, 3, 300, 128), (1, 4, 1000, 64), (2, 8, 4097, 128),
             (1, 12, 2049, 128), (1, 1, 70000, 128), (3, 5, 513, 32)]


@pytest.mark.parametrize("B,H,L,d", DEC_SMALL)
def test_decode_small(alibi, B, H, L, d):
    rng_seed = B * 100 + L
    q, kc, vc = W.gaussian_qkv_bf16((B, H, d), seed=rng_seed, kv_shape=(B, H, L, d))
    ref = oracle.decode_ref(q, kc, vc, oracle.slopes_ref(H))
    out = alibi.attn_decode(dev(q), dev(kc), dev(vc), alibi.slopes(H))
    check_bf16(out, ref, f"decode B{B} H{H} L{L} d{d}")


def test_decode_equals_last_forward_row(alibi):
    B, H, N, d = 1, 8, 777, 128
    q, k, v = W.gaussian_qkv_bf16((B, H, N, d), seed=21)
    s = alibi.slopes(H)
    full = alibi.attn_fwd(dev(q), dev(k), dev(v), s, causal=True)
    dq = dev(q[:, :, -1, :])
    dec = alibi.attn_decode(dq, dev(k), dev(v), s)
    ref = oracle.decode_ref(q[:, :, -1, :], k, v, oracle.slopes_ref(H))
    check_bf16(dec, ref, "decode vs oracle")
    check_bf16(full[:, :, -1, :], ref, "forward last row vs oracle")
    diff = (dec.float() - full[:, :, -1, :].float()).abs().max().item()
    print(f"[parity] decode vs forward last row: {diff:.3e}", flush=True)
    assert diff <= 2 * BF16_TOL


def test_fwd_far_key_dominates_rows(alibi, fwd_form):
    # A key far behind the diagonal scores far above every nearer key (q_i . k_j
    # large), so an off-diagonal tile must raise the running maximum well past
    # what the diagonal set: the rare rescale-and-redo path of the kernel.
    B, H, N, d = 1, 2, 1500, 128
    q, k, v = W.gaussian_qkv_f32((B, H, N, d), seed=41)
    q[:, :, 1200:1300] = k[:, :, 10:11] * 3.0      # rows 1200..1299 align with key 10
    qb, kb, vb = (W.to_bf16_tensor(x) for x in (q, k, v))
    s = np.array([0.01, 0.001], dtype=np.float32)
    out = alibi.attn_fwd(dev(qb), dev(kb), dev(vb), torch.from_numpy(s), causal=True)
    ref = oracle.attn_ref(qb, kb, vb, s, causal=True)
    check_bf16(out, ref, "far key dominates")


@pytest.mark.parametrize("B,H,L,d", [(2, 3, 300, 128), (1, 1, 70000, 128), (3, 5, 513, 32), (64, 64, 40, 64)])
def test_decode_caller_workspace_matches_library_workspace(alibi, B, H, L, d):
    # the same kernels on a workspace the caller owns: bitwise-equal output
    q, kc, vc = W.gaussian_qkv_bf16((B, H, d), seed=B * 7 + L, kv_shape=(B, H, L, d))
    s = alibi.slopes(H)
    qd, kd, vd = dev(q), dev(kc), dev(vc)
    need = alibi.decode_ws_bytes(B, H, L, d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda") if need > 0 else None
    a = alibi.attn_decode(qd, kd, vd, s)
    b = alibi.attn_decode_ws(qd, kd, vd, ws, s)
    torch.cuda.synchronize()
    print(f"[parity] decode ws B{B} H{H} L{L} d{d}: {need} workspace bytes", flush=True)
    assert torch.equal(a, b)
    check_bf16(b, oracle.decode_ref(q, kc, vc, oracle.slopes_ref(H)), f"decode ws B{B} H{H} L{L} d{d}")


def test_decode_caller_workspaces_on_two_streams(alibi):
    # two decodes in flight at once on two streams, each with its own workspace
    shapes = [(2, 4, 9000, 128, 61), (1, 8, 20000, 64, 62)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs, refs = [], []
    for (B, H, L, d, seed), st in zip(shapes, streams):
        q, kc, vc = W.gaussian_qkv_bf16((B, H, d), seed=seed, kv_shape=(B, H, L, d))
        refs.append(oracle.decode_ref(q, kc, vc, oracle.slopes_ref(H)))
        qd, kd, vd = dev(q), dev(kc), dev(vc)
        ws = torch.empty(max(alibi.decode_ws_bytes(B, H, L, d), 16), dtype=torch.uint8, device="cuda")
        sl = alibi.slopes(H).cuda()
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            outs.append((alibi.attn_decode_ws(qd, kd, vd, ws, sl), ws, qd, kd, vd, sl))
    torch.cuda.synchronize()
    for (o, *_), ref, (B, H, L, d, _) in zip(outs, refs, shapes):
        check_bf16(o, ref, f"decode ws two streams B{B} H{H} L{L} d{d}")
