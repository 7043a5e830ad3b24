"""Exact underflow skipping in the decode (needs an MI355X).

With a KV cache the query sits at position L - 1; every score is at most
|q| max|k| / sqrt(d) - m_h D and the newest key's is at least -|q| max|k| / sqrt(d),
so keys far enough back have weights that round to exactly zero ("When
Attention Goes Blind", Sec. 3.3 and 5.1-5.2). alibi_attn_decode_ex skips them,
and the tests hold it to the unskipped decode bit for bit, and to the fp64
oracle as every decode is. The key-norm bound comes from alibi_key_norm_max,
checked against norms computed on the host.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity_util import check_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def alibi():
    import alibi_linear_position_amd as mod
    mod.load_library()
    return mod


def _cache(B, H, L, d, seed):
    kc = W.device_gaussian_bf16((B, H, L, d), seed=seed)
    vc = W.device_gaussian_bf16((B, H, L, d), seed=seed + 1)
    q = W.device_gaussian_bf16((B, H, d), seed=seed + 2)
    return q, kc, vc


@pytest.mark.parametrize("B,H,L,d", [(2, 3, 1000, 64), (1, 4, 4097, 128), (3, 2, 1, 128)])
def test_key_norm_max_matches_host(alibi, B, H, L, d):
    _, kc, _ = _cache(B, H, L, d, 5)
    got = alibi.key_norm_max(kc).cpu().double().numpy()
    want = np.sqrt((kc.cpu().double().numpy() ** 2).sum(-1)).max(-1)
    err = np.abs(got - want) / want
    print(f"[parity] key_norm_max B{B} H{H} L{L} d{d}: max rel err {err.max():.2e}", flush=True)
    assert np.all(err <= 1e-6)


# (B, H, L, d, slope recipe): the c5 heads at two batches, the steep recipe
# (most keys skipped), a ragged length, an unsplit plan (B H = 4096: one
# workgroup per (b, h)) and a d the MFMA kernels do not take
CASES = [
    (2, 32, 32768, 128, "default"),
    (1, 8, 5000, 64, "steep"),
    (4, 16, 2049, 128, "steep"),
    (64, 64, 700, 128, "default"),
    (2, 4, 3000, 96, "steep"),
]


def _slopes(recipe, H):
    return oracle.slopes_ref(H) if recipe == "default" else oracle.slopes_recipe_ref(recipe, H, False)


@pytest.mark.parametrize("B,H,L,d,recipe", CASES, ids=lambda x: str(x))
def test_decode_skip_is_bitwise_the_decode(alibi, B, H, L, d, recipe):
    q, kc, vc = _cache(B, H, L, d, 11)
    s = torch.from_numpy(_slopes(recipe, H)).float()
    if d in (64, 128):
        kn = alibi.key_norm_max(kc)
    else:  # a bound computed by the caller, as alibi_key_norm_max would give it
        kn = kc.float().norm(dim=-1).amax(dim=-1).contiguous()
    full = alibi.attn_decode(q, kc, vc, s)
    skip = alibi.attn_decode_ex(q, kc, vc, s, skip_underflow=True, key_norm_max=kn)
    torch.cuda.synchronize()
    diff = (full.float() - skip.float()).abs().max().item()
    print(f"[parity] decode skip B{B} H{H} L{L} d{d} {recipe}: max |skip - full| = {diff}", flush=True)
    assert torch.equal(full.view(torch.int16), skip.view(torch.int16))
    if B * H * L <= 4 * 32 * 5000:
        st = oracle.slopes_ref(H) if recipe == "default" else oracle.slopes_recipe_ref(recipe, H, False)
        ref = oracle.decode_ref(q.cpu(), kc.cpu(), vc.cpu(), st)
        check_bf16(skip, ref, f"decode skip B{B} H{H} L{L} d{d} {recipe} vs oracle")


def test_decode_skip_never_reads_dead_keys(alibi):
    # A NaN planted in V far behind the query of the steepest head: the plain
    # decode reads it and its weight 0 times NaN poisons that head's output;
    # the skipping decode never reads that key, so the head stays finite and
    # every other head is bit for bit the plain decode's.
    B, H, L, d = 1, 8, 20000, 128
    q, kc, vc = _cache(B, H, L, d, 21)
    s = torch.from_numpy(oracle.slopes_ref(H)).float()   # head 0: m = 2^-1
    vc[0, 0, 1000] = float("nan")                         # 18999 keys behind the query
    kn = alibi.key_norm_max(kc)
    full = alibi.attn_decode(q, kc, vc, s)
    skip = alibi.attn_decode_ex(q, kc, vc, s, skip_underflow=True, key_norm_max=kn)
    torch.cuda.synchronize()
    print(f"[parity] decode with a NaN far back: plain head 0 finite={bool(torch.isfinite(full[0, 0]).all())}, "
          f"skipping head 0 finite={bool(torch.isfinite(skip[0, 0]).all())}", flush=True)
    assert not torch.isfinite(full[0, 0]).all()
    assert torch.isfinite(skip[0, 0]).all()
    assert torch.equal(full[0, 1:].view(torch.int16), skip[0, 1:].view(torch.int16))
    vc[0, 0, 1000] = 0.0
    clean = alibi.attn_decode(q, kc, vc, s)
    assert torch.equal(clean[0, 0].view(torch.int16), skip[0, 0].view(torch.int16))


def test_decode_ex_without_options_is_the_decode(alibi):
    q, kc, vc = _cache(2, 4, 3000, 128, 31)
    s = torch.from_numpy(oracle.slopes_ref(4)).float()
    a = alibi.attn_decode(q, kc, vc, s)
    b = alibi.attn_decode_ex(q, kc, vc, s)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
