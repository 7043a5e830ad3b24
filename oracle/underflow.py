"""Softmax-underflow diagnostics for ALiBi (test infrastructure, not the product).

Source: "When Attention Goes Blind: Numerical Failure in ALiBi Positional
Encodings" (arXiv 2608.03994): Sec. 3.2 (threshold tau_u with e^x = 0 below
it; blindness distance Delta_h(eps) = min{d : eps - m_h d <= tau_u},
delta_h = Delta_h(0)); Sec. 3.3 (share of underflowed entries, Fig. 1b);
Sec. 3.4 "Log-scaled Distances" (D* = log(D + 1)); App. A, Table 4 (format
thresholds); Table 1 and App. F, Table 8 (expected blindness distances,
rounded to the nearest integer); Sec. 5.2 (a steep head as a window).

Reading of the pages: the text defines delta with tau_u, but every printed
delta and share reproduces only with the denormal threshold tau_d = ln 2^-126
(|tau_d| = 87.3365) and rounding to nearest. Both thresholds are available
here; callers choose.
"""
from __future__ import annotations

import math

import numpy as np


def format_thresholds(fmt: str) -> dict:
    """Underflow / denormal / overflow thresholds of exp() in a float format.

    Derived from the format's parameters (not from the printed table):
    tau_u = ln(smallest subnormal), tau_d = ln(smallest normal),
    tau_o = ln(largest finite). ``fmt`` is "bf16" or "fp32" (Table 4's rows).
    """
    import torch
    dt = {"bf16": torch.bfloat16, "fp32": torch.float32}[fmt]
    fi = torch.finfo(dt)
    tiny = float(fi.tiny)               # smallest normal
    sub = tiny * float(fi.eps)          # smallest subnormal: one ulp below the normals
    return {"tau_u": math.log(sub), "tau_d": math.log(tiny), "tau_o": math.log(float(fi.max))}


def blindness_distance(m: float, eps: float, tau: float) -> int:
    """Delta(eps) = the least natural d with eps - m d <= tau (Sec. 3.2)."""
    if m <= 0:
        raise ValueError("slope must be positive")
    d = max(0, math.ceil((eps - tau) / m))
    # guard the ceil against rounding at exact multiples
    while d > 0 and eps - m * (d - 1) <= tau:
        d -= 1
    while eps - m * d > tau:
        d += 1
    return d


def expected_blindness_distance(m: float, tau: float) -> float:
    """The real-valued crossing distance -tau / m (Table 1 / Table 8 round it to nearest)."""
    return -tau / m


def log_scaled_blindness_distance(m: float, tau: float) -> float:
    """Distance at which -m log(D + 1) reaches tau (Sec. 3.4, log-scaled distances)."""
    return math.exp(-tau / m) - 1.0


def underflow_fraction_by_distance(slopes, n_dist: int, tau: float) -> float:
    """Share of (head, distance) pairs, distances 0..n_dist-1, with bias at or past tau (A = 0).

    This is the quantity of Fig. 1b read at one token distance: the mean over
    heads of the share of distances whose bias -m d has crossed tau.
    """
    s = np.asarray(slopes, dtype=np.float64).reshape(-1, 1)
    d = np.arange(n_dist, dtype=np.float64).reshape(1, -1)
    return float(np.mean(-s * d <= tau))


def underflow_fraction_causal(m: float, n: int, tau: float) -> float:
    """Share of the causal triangle (diagonal included) whose bias has crossed tau (A = 0).

    The convention of Sec. 5.2 (a steep head's window against a 2048 context).
    Counted in closed form per distance: distance t occurs n - t times.
    """
    t = np.arange(n, dtype=np.float64)
    count = n - t
    hit = (-float(m) * t) <= tau
    return float(np.sum(count * hit) / np.sum(count))


def underflow_fraction_data(q, k, m: float, tau, rows=None, causal=True):
    """Data-dependent share of causal entries whose stable-softmax exponent is <= tau.

    For row i the exponent is x_ij = s_ij - max_j s_ij with s_ij the biased
    scaled score (Table 4's condition x <= tau_u). Returns the share over the
    chosen rows' causal entries and over the last chosen row alone. q, k: one
    head, (N, d), any float type (upcast to fp64). ``tau`` may be a sequence
    of thresholds: then one such dict per threshold, in order, from one pass.
    """
    taus = [float(tau)] if np.isscalar(tau) else [float(t) for t in tau]
    import torch
    qf = q.detach().to("cpu", torch.float64).numpy() if isinstance(q, torch.Tensor) else np.asarray(q, np.float64)
    kf = k.detach().to("cpu", torch.float64).numpy() if isinstance(k, torch.Tensor) else np.asarray(k, np.float64)
    n, dk = qf.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    hit = [0] * len(taus)
    tot = 0
    last_share = [0.0] * len(taus)
    for i in rows:
        nk = int(i) + 1 if causal else kf.shape[0]
        s = (kf[:nk] @ qf[i]) / math.sqrt(dk)
        s = s - float(m) * np.abs(int(i) - np.arange(nk, dtype=np.float64))
        x = s - np.max(s)
        for t, tv in enumerate(taus):
            h = int(np.sum(x <= tv))
            hit[t] += h
            last_share[t] = h / nk
        tot += nk
    res = [{"share": hit[t] / tot, "last_row_share": last_share[t]} for t in range(len(taus))]
    return res[0] if np.isscalar(tau) else res
