"""Tolerance checks shared by the GPU parity tests (no GPU needed to import).

* fp32 path: max |gpu - oracle| <= 1e-5.
* bf16 paths: every element satisfies |gpu - o| <= 1e-2 + ulp_bf16(o) / 2, where
  o is the fp64 oracle value: the bf16 output can only land on the bf16 grid,
  so half an ulp of rounding is granted on top of the 1e-2 compute budget (it
  matters only for |o| >= 2). The raw max |gpu - o| is printed too.
"""
import numpy as np
import torch

import oracle

BF16_TOL = 1e-2
F32_TOL = 1e-5
U_BF16 = 2.0 ** -8  # unit roundoff of bf16: 8 significant bits, round to nearest even
# The forward's row log-sum-exp: its running maximum plus the log of a row sum of
# bf16-rounded weights, a sum of positive terms each within relative U_BF16, so
# |err| <= ln(1 + 2^-8) = 3.90e-3 plus fp32 rounding.
LSE_TOL = 4e-3
# Gradients: |gpu - o| <= G_ATOL + G_RTOL (|o| + M) + E per element, the bar
# derived in tests/test_gpu_backward.py.
G_ATOL = 1e-2
G_RTOL = 1e-2


def o_rounding_bound(p, o, q, k, do):
    """Bound on what the bf16 rounding of the forward output O does to dq and dk.

    The backward takes D_i = sum_c dO_ic O_ic from the stored bf16 output, so
    |dD_i| <= U_BF16 sum_c |dO_ic| |O_ic|. D enters dS = P (dP - D) as the term
    -P_ij dD_i, hence |delta dq_i| <= |dD_i| sum_j P_ij |K_j| / sqrt(d) and
    |delta dk_j| <= sum_i P_ij |dD_i| |Q_i| / sqrt(d). Cancellation inside dS
    does not shrink this term: where P is nearly one-hot (a steep head with
    log-scaled distances) the true dS is tiny and this rounding dominates it.
    All arguments are fp64 arrays of one head: p (n, n), o, q, k, do (n, d).
    """
    scale = 1.0 / np.sqrt(q.shape[-1])
    dd = U_BF16 * np.sum(np.abs(do) * np.abs(o), axis=-1, keepdims=True)
    pd = p * dd
    return pd @ np.abs(k) * scale, pd.T @ np.abs(q) * scale


def half_ulp_bf16(o):
    o = np.abs(np.asarray(o, dtype=np.float64))
    _, e = np.frexp(o)  # o = m 2^e, m in [0.5, 1)
    h = np.ldexp(1.0, e - 9)
    return np.where(o > 0, h, 0.0)


def check_bf16(gpu, ref, label):
    g = gpu.detach().to("cpu", torch.float64).numpy()
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{label}: non-finite output"
    err = np.abs(g - ref)
    allowed = BF16_TOL + half_ulp_bf16(ref)
    bad = int(np.sum(err > allowed))
    needed_ulp = int(np.sum(err > BF16_TOL))
    print(f"[parity] {label}: max|err|={err.max():.3e} elements>1e-2={needed_ulp} failing={bad}", flush=True)
    assert bad == 0, f"{label}: {bad} elements beyond tolerance, max err {err.max()}"
    return float(err.max())


class Bf16Stats:
    """The bf16 bar of check_bf16 accumulated over the pieces of one large
    configuration (one (b, h) at a time keeps host memory bounded)."""

    def __init__(self, label):
        self.label, self.max_err, self.over, self.failing, self.n = label, 0.0, 0, 0, 0

    def add(self, gpu, ref):
        g = gpu.detach().to("cpu", torch.float64).numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu)
        ref = np.asarray(ref, dtype=np.float64)
        assert g.shape == ref.shape, (g.shape, ref.shape)
        assert np.all(np.isfinite(g)), f"{self.label}: non-finite output"
        err = np.abs(g - ref)
        self.max_err = max(self.max_err, float(err.max()))
        self.over += int(np.sum(err > BF16_TOL))
        self.failing += int(np.sum(err > BF16_TOL + half_ulp_bf16(ref)))
        self.n += err.size

    def finish(self):
        print(f"[parity] {self.label}: {self.n} elements, max|err|={self.max_err:.3e} "
              f"elements>1e-2={self.over} failing={self.failing}", flush=True)
        assert self.failing == 0, f"{self.label}: {self.failing} elements beyond tolerance, max err {self.max_err}"
        return self.max_err


def dev(x):
    return x.to("cuda").contiguous()


def check_grad(gpu, ref, label, mag=None, extra=0.0):
    """mag: the oracle's magnitude sums for these elements (None: |ref| bounds them);
    extra: the bound E on the effect of the output's bf16 rounding."""
    g = gpu.detach().to("cpu", torch.float64).numpy()
    err = np.abs(g - ref)
    m = np.abs(ref) if mag is None else np.asarray(mag)
    bar = G_ATOL + G_RTOL * (np.abs(ref) + m) + extra
    bad = int(np.sum(err > bar))
    over_old = int(np.sum(err > G_ATOL + G_RTOL * np.abs(ref)))
    print(f"[parity] {label}: max|err|={err.max():.3e} max|ref|={np.abs(ref).max():.3e} "
          f"max err/bar={np.max(err / bar):.3f} beyond 1e-2+1e-2|o|: {over_old} failing={bad}", flush=True)
    assert np.all(np.isfinite(g)) and bad == 0, label


def check_grads(gpu3, q, k, v, do, m, causal, label, clamp=None, log_distance=False, softcap=None):
    """dq, dk, dv of one head (bf16 tensors) against the fp64 oracle's chain rule."""
    (rq, rk, rv), (mq, mk, mv) = oracle.attn_backward_head_ref(q, k, v, do, m, causal, magnitudes=True,
                                                               clamp=clamp, log_distance=log_distance,
                                                               softcap=softcap)
    o, p = oracle.variant_head_ref(q, k, v, m, causal, clamp=clamp, log_distance=log_distance, softcap=softcap)
    eq, ek = o_rounding_bound(p, o, *(x.double().numpy() for x in (q, k, do)))
    for g, r, mg, e, n in zip(gpu3, (rq, rk, rv), (mq, mk, mv), (eq, ek, 0.0), ("dq", "dk", "dv")):
        check_grad(g, r, f"{n} {label}", mg, e)
