"""Tolerance checks shared by the GPU parity tests (no GPU needed to import).

* fp32 path: max |gpu - oracle| <= 1e-5.
* bf16 paths: every element satisfies |gpu - o| <= 1e-2 + ulp_bf16(o) / 2, where
  o is the fp64 oracle value: the bf16 output can only land on the bf16 grid,
  so half an ulp of rounding is granted on top of the 1e-2 compute budget (it
  matters only for |o| >= 2). The raw max |gpu - o| is printed too.
"""
import numpy as np
import torch

BF16_TOL = 1e-2
F32_TOL = 1e-5


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


def dev(x):
    return x.to("cuda").contiguous()
