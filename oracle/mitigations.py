"""Underflow mitigations of ALiBi in plain fp64 (test infrastructure, not the product).

Source: "When Attention Goes Blind: Numerical Failure in ALiBi Positional
Encodings" (arXiv 2608.03994):

* Sec. 3.4 "Clamping": the bias is floored at a constant, B* = max(B, c_clamp).
* Sec. 3.4 "Robust Slopes" and Sec. 4.2: slopes chosen from target blindness
  distances delta_h; App. F, Table 8 lists the targets of the trained models.
* Sec. 3.4 "Log-scaled Distances": D* = log(D + 1) replaces the distance.
* Sec. 3.4 "Soft Capping": the content logits (not the bias) become
  A* = z tanh(A / z).
* Sec. 4.3: the settings used there (c_clamp = -87, z = 50) and the slopes
  of the explicit recipe adapted to log distances, m_h = -tau / log(delta_h + 1).
* Sec. 5.2 "Connection to Previous Work" and Sec. 5.3 "Recommendations for
  Model Training": a hard sliding window as the alternative to clamping, which
  lets the computation ignore the out-of-window entries.

Readings (where the pages leave a step open):

* The threshold behind every printed delta is the fp32 denormal limit
  tau_d = ln 2^-126 (|tau_d| = 87.3365); a slope for a target distance is
  therefore m = |tau_d| / delta.
* Between the first and the last target the distances are spaced
  geometrically, delta_h = delta_1 (delta_H / delta_1)^(h / (H - 1)), which
  reproduces every row of Table 8 for H = 9 (the doubling rows included).
* The explicit recipe doubles from 32 (32, 64, ...), as in Table 8; Sec. 4.3's
  "delta_H = 4096" for the trained models disagrees with Table 8's 8192 and is
  not used.
* Heads are ordered steepest first (delta_1 is the smallest distance), like the
  default geometric schedule.
* The hard window of a head is a count of tokens, W_h: key j stays visible to
  query i when 0 <= i - j < W_h (positions, causal form only), so W_h = 1
  keeps the query's own key and W_h <= 0 none. This count reproduces Sec.
  5.2's figure (a 124-token window in a 2048-token context leaves 88.3% of
  the causal entries out). The pages fix no window per head, so W_h is an
  argument; the natural choice is the head's blindness distance.
* The order of operations per entry is the one the four equations imply:
  A = Q K^T / sqrt(d); A <- z tanh(A / z) if soft-capped; D = i - j (|i - j|
  without the causal mask); D <- log(D + 1) if log-scaled; B = -m D;
  B <- max(B, c_clamp) if clamped; logits = A + B; causal mask; softmax; times V.
"""
from __future__ import annotations

import math

import numpy as np

from .alibi_ref import _f64, distance_ref, softmax_rows_ref

#: |ln 2^-126|: the threshold the printed blindness distances follow
TAU_D = 126.0 * math.log(2.0)

#: first and last target blindness distance of each slope recipe (Sec. 4.2,
#: Sec. 3.4 "Robust Slopes", Table 8)
RECIPE_ENDPOINTS = {
    "steep": (128.0, 512.0),
    "safe": (2048.0, 4096.0),
    "wide": (16.0, 4096.0),
}


def recipe_distances(recipe: str, H: int) -> np.ndarray:
    """Target blindness distances delta_1..delta_H of a slope recipe (fp64)."""
    if H < 1:
        raise ValueError("H must be >= 1")
    if recipe == "explicit":
        return np.array([32.0 * 2.0 ** h for h in range(H)], dtype=np.float64)
    lo, hi = RECIPE_ENDPOINTS[recipe]
    if H == 1:
        return np.array([lo], dtype=np.float64)
    return np.array([lo * (hi / lo) ** (h / (H - 1)) for h in range(H)], dtype=np.float64)


def slopes_recipe_ref(recipe: str, H: int, log_distance: bool = False) -> np.ndarray:
    """Slopes (fp32, RNE from fp64) whose blindness distances are the recipe's targets.

    Linear distances: m_h = |tau_d| / delta_h, so -m_h delta_h = tau_d.
    With log-scaled distances (Sec. 4.3): m_h = |tau_d| / log(delta_h + 1), so
    the bias reaches tau_d at the same distance delta_h.
    """
    dl = recipe_distances(recipe, H)
    if log_distance:
        m = TAU_D / np.array([math.log(x + 1.0) for x in dl])
    else:
        m = TAU_D / dl
    return m.astype(np.float32)


def variant_head_ref(q, k, v, m, causal=True, clamp=None, log_distance=False, softcap=None,
                     q_pos0=0, k_pos0=0, window=None):
    """One head with any mix of the Sec. 3.4 mitigations; returns (out, weights) in fp64.

    q: (n_q, d), k: (n_k, d), v: (n_k, d_v). Query row r sits at position
    q_pos0 + r and key row c at k_pos0 + c. A row with no visible key gives 0.
    window: the head's hard window of W tokens (Sec. 5.2-5.3; causal only): key
    c stays visible to row r when 0 <= dist < W; None = no window.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    a = (q @ k.T) / math.sqrt(q.shape[-1])
    if softcap is not None:
        a = float(softcap) * np.tanh(a / float(softcap))
    dist = distance_ref(q.shape[0], k.shape[0], q_pos0, k_pos0)
    visible = dist >= 0 if causal else np.ones(dist.shape, dtype=bool)
    if window is not None:
        if not causal:
            raise ValueError("the hard window is defined for the causal form only")
        visible = visible & (dist < int(window))
    dd = np.abs(dist).astype(np.float64)   # equals i - j wherever a causal key is visible
    if log_distance:
        dd = np.log(dd + 1.0)
    bias = -float(m) * dd
    if clamp is not None:
        bias = np.maximum(bias, float(clamp))
    logits = np.where(visible, a + bias, -np.inf)
    w = softmax_rows_ref(logits)
    return w @ v, w


def variant_ref(q, k, v, slopes, causal=True, clamp=None, log_distance=False, softcap=None,
                q_offset=0, k_offset=0, return_weights=False, windows=None):
    """Multi-head form of :func:`variant_head_ref`.

    q: (B, H, n_q, d); k, v: (B, H, n_k, d). windows: None or H per-head hard
    windows. Returns out (B, H, n_q, d_v), fp64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, H = q.shape[0], q.shape[1]
    slopes = np.asarray(_f64(slopes)).reshape(-1)
    out = np.empty((B, H, q.shape[2], v.shape[-1]), dtype=np.float64)
    wts = np.empty((B, H, q.shape[2], k.shape[2]), dtype=np.float64) if return_weights else None
    for b in range(B):
        for h in range(H):
            o, w = variant_head_ref(q[b, h], k[b, h], v[b, h], slopes[h], causal, clamp,
                                    log_distance, softcap, q_offset, k_offset,
                                    None if windows is None else int(windows[h]))
            out[b, h] = o
            if return_weights:
                wts[b, h] = w
    return (out, wts) if return_weights else out
