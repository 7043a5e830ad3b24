"""Plain fp64 definitions of ALiBi attention (test infrastructure, not the product).

Sources (web pages, cited by title and section):

* "ALiBi: Attention with Linear Biases" (abhik.ai) -- sections "From distance
  to a normalized weight", "Different heads, different distance penalties",
  "The mask and the bias have different jobs", and the KV-cache remark after
  the full-sequence example.
* "ALiBi and Relative Position Bias" (quantmemo.com) -- "The mechanics": the
  symmetric score q.k/sqrt(d) - m|i-j|.
* "When Attention Goes Blind: Numerical Failure in ALiBi Positional Encodings"
  (arXiv 2608.03994) -- Sec. 3.1, Eq. 1-3 (A = QK^T/sqrt(d_k), B = -m D,
  D = (i-j) for j < i); Sec. 3.2, Eq. 4 (softmax); App. B.1 (stable softmax).
* "ALiBi in Attention: Complete Implementation" (mbrenndoerfer.com) -- the
  ``alibi_attention(Q, K, V, slopes, causal)`` description: per-head bias from
  absolute distances, optional causal mask of the strict upper triangle, stable
  softmax, NaN rows set to zero, weights times V.
* "ALiBi: give a Transformer position sense with one line" (dev.to) --
  "Per-head slopes form a geometric ladder" and "One matrix: -m(i-j)".

Everything is computed in float64. Inputs given in fp32 or bf16 are upcast
exactly, so the oracle sees the very values the device sees.
"""
from __future__ import annotations

import math

import numpy as np


# ---------------------------------------------------------------------------
# Slopes
# ---------------------------------------------------------------------------

def slopes_pow2_ref(n: int) -> np.ndarray:
    """Geometric schedule for a power-of-two head count, in fp64.

    Head h (counted from zero) gets 2^(-8(h+1)/n): the first slope is 2^(-8/n)
    and each next one is smaller by the same ratio 2^(-8/n) ("Different heads,
    different distance penalties", abhik.ai; "Per-head slopes form a geometric
    ladder", dev.to). The power is evaluated in fp64, where it is exact for
    every n that divides 8 and correctly rounded otherwise.
    """
    return np.array([2.0 ** (-8.0 * (h + 1) / n) for h in range(n)], dtype=np.float64)


def slopes_ref(H: int) -> np.ndarray:
    """Per-head ALiBi slopes as fp32 (round to nearest even from fp64).

    Power-of-two H: the geometric schedule of :func:`slopes_pow2_ref`.
    Otherwise (abhik.ai, "Different heads, different distance penalties"): take
    the schedule of c = the largest power of two below H, then append entries
    0, 2, 4, ... of the schedule for 2c until H slopes are listed. The order is
    kept (not sorted), so the six-head list is 0.25, 0.0625, 0.015625,
    0.00390625, 0.5, 0.125.
    """
    if H < 1:
        raise ValueError("H must be >= 1")
    c = 1 << (H.bit_length() - 1)
    if c == H:
        s = slopes_pow2_ref(H)
    else:
        extra = slopes_pow2_ref(2 * c)[0::2][: H - c]
        s = np.concatenate([slopes_pow2_ref(c), extra])
    return s.astype(np.float32)


# ---------------------------------------------------------------------------
# Distance, bias, softmax
# ---------------------------------------------------------------------------

def distance_ref(n_q: int, n_k: int, q_pos0: int = 0, k_pos0: int = 0) -> np.ndarray:
    """Signed distance i - j between query and key *positions* (int64 matrix).

    Query row r sits at position q_pos0 + r and key column c at k_pos0 + c, so
    a KV-cache query is placed at its real sequence position rather than at
    zero (abhik.ai, the remark after the full-sequence example).
    """
    i = np.arange(n_q, dtype=np.int64)[:, None] + q_pos0
    j = np.arange(n_k, dtype=np.int64)[None, :] + k_pos0
    return i - j


def bias_ref(m: float, dist: np.ndarray, causal: bool) -> np.ndarray:
    """ALiBi bias in fp64.

    causal: -m (i - j) (Eq. 2-3 of "When Attention Goes Blind"; dev.to "One
    matrix"); entries with j > i are masked separately and their value here is
    irrelevant.  Not causal: the symmetric -m |i - j| of quantmemo.com "The
    mechanics" and of mbrenndoerfer.com's ``distances = abs(...)``.
    """
    d = dist.astype(np.float64)
    if not causal:
        d = np.abs(d)
    return -float(m) * d


def softmax_rows_ref(x: np.ndarray) -> np.ndarray:
    """Stable row softmax (App. B.1 of "When Attention Goes Blind").

    Subtract the row maximum, exponentiate, divide by the row sum. A row whose
    entries are all -inf yields NaN, which is replaced by 0 as in
    mbrenndoerfer.com's implementation.
    """
    with np.errstate(invalid="ignore"):
        mx = np.max(x, axis=-1, keepdims=True)
        e = np.exp(x - mx)
        w = e / np.sum(e, axis=-1, keepdims=True)
    return np.nan_to_num(w, nan=0.0)


def _f64(a) -> np.ndarray:
    """Exact upcast of an fp32/bf16 numpy array or torch tensor to fp64 numpy."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is present in this image
        pass
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def attn_head_ref(q, k, v, m, causal=True, q_pos0=0, k_pos0=0):
    """One head: returns (out (n_q, d_v), weights (n_q, n_k)), fp64.

    Steps, in the order of Eq. 1 of "When Attention Goes Blind":
    A = Q K^T / sqrt(d_k); add the bias -m D; mask future keys with -inf
    when causal (abhik.ai, "From distance to a normalized weight"); stable
    softmax per row; multiply by V.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    dk = q.shape[-1]
    a = (q @ k.T) / math.sqrt(dk)
    dist = distance_ref(q.shape[0], k.shape[0], q_pos0, k_pos0)
    logits = a + bias_ref(m, dist, causal)
    if causal:
        logits = np.where(dist < 0, -np.inf, logits)
    w = softmax_rows_ref(logits)
    return w @ v, w


def attn_ref(q, k, v, slopes, causal=True, return_weights=False):
    """Full multi-head attention, fp64, materialising every (N, N) bias.

    q, k, v: (B, H, N, d) or (H, N, d); slopes: H values (used exactly as given,
    normally the fp32 values of :func:`slopes_ref`). Returns out in fp64 with
    q's leading shape, plus the (.., N, N) weights when asked.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    squeeze = q.ndim == 3
    if squeeze:
        q, k, v = q[None], k[None], v[None]
    B, H, N, _ = q.shape
    slopes = np.asarray(_f64(slopes)).reshape(-1)
    if slopes.shape[0] != H:
        raise ValueError("one slope per head expected")
    out = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    wts = np.empty((B, H, N, k.shape[2]), dtype=np.float64) if return_weights else None
    for b in range(B):
        for h in range(H):
            o, w = attn_head_ref(q[b, h], k[b, h], v[b, h], slopes[h], causal)
            out[b, h] = o
            if return_weights:
                wts[b, h] = w
    if squeeze:
        out = out[0]
        wts = None if wts is None else wts[0]
    return (out, wts) if return_weights else out


def attn_rows_ref(q_bh, k_bh, v_bh, m, rows, causal=True):
    """Selected output rows of one head, fp64 (for sequences too long to materialise).

    Each requested query row i is computed from its own bias row -m (i - j)
    over all keys, exactly as the full definition would, so sampled rows of a
    16384-token head cost O(N d) each.
    """
    q = _f64(q_bh)
    k = _f64(k_bh)
    v = _f64(v_bh)
    rows = np.asarray(rows, dtype=np.int64)
    n_k = k.shape[0]
    dk = q.shape[-1]
    out = np.empty((rows.shape[0], v.shape[-1]), dtype=np.float64)
    for t, i in enumerate(rows):
        a = (k @ q[i]) / math.sqrt(dk)
        dist = distance_ref(1, n_k, int(i), 0)[0]
        logit = a + bias_ref(m, dist, causal)
        if causal:
            logit = np.where(dist < 0, -np.inf, logit)
        w = softmax_rows_ref(logit[None, :])[0]
        out[t] = w @ v
    return out


def decode_ref(q, kcache, vcache, slopes, pairs=None):
    """Single-query decode over a KV cache, fp64.

    q: (B, H, d); caches: (B, H, L, d). The query is the newest token, at
    position L - 1, and key j keeps its real position j, so the bias is
    -m_h (L - 1 - j) and no key is in the future (abhik.ai, KV-cache remark).
    ``pairs`` optionally restricts the work to a list of (b, h); the result is
    then an array of shape (len(pairs), d).
    """
    slopes = np.asarray(_f64(slopes)).reshape(-1)
    if pairs is None:
        B, H = q.shape[0], q.shape[1]
        pairs_ = [(b, h) for b in range(B) for h in range(H)]
    else:
        pairs_ = list(pairs)
    res = []
    for b, h in pairs_:
        qb = _f64(q[b, h])
        kb = _f64(kcache[b, h])
        vb = _f64(vcache[b, h])
        L = kb.shape[0]
        a = (kb @ qb) / math.sqrt(qb.shape[0])
        logit = a + bias_ref(slopes[h], distance_ref(1, L, L - 1, 0)[0], True)
        w = softmax_rows_ref(logit[None, :])[0]
        o = w @ vb
        res.append(o)
    res = np.stack(res)
    if pairs is None:
        res = res.reshape(q.shape[0], q.shape[1], -1)
    return res


def attn_bruteforce(q, k, v, slopes, causal=True):
    """Pure-Python triple loop (no BLAS, no numpy arithmetic) for tiny inputs.

    Each weight is exp(s_ij - max_j s_ij) / sum, with s_ij the scaled dot
    product minus m |i - j| (or -inf for a future key when causal). Shapes
    (H, N, d). Returns (out, weights) as nested Python float lists.
    """
    qf = _f64(q).tolist()
    kf = _f64(k).tolist()
    vf = _f64(v).tolist()
    sl = [float(x) for x in np.asarray(_f64(slopes)).reshape(-1)]
    H = len(qf)
    out, wts = [], []
    for h in range(H):
        n_q, n_k, dk, dv = len(qf[h]), len(kf[h]), len(qf[h][0]), len(vf[h][0])
        oh, wh = [], []
        for i in range(n_q):
            s = []
            for j in range(n_k):
                if causal and j > i:
                    s.append(None)
                    continue
                dot = 0.0
                for t in range(dk):
                    dot += qf[h][i][t] * kf[h][j][t]
                s.append(dot / math.sqrt(dk) - sl[h] * abs(i - j))
            mx = max(x for x in s if x is not None)
            e = [0.0 if x is None else math.exp(x - mx) for x in s]
            tot = sum(e)
            w = [x / tot for x in e]
            o = [sum(w[j] * vf[h][j][t] for j in range(n_k)) for t in range(dv)]
            oh.append(o)
            wh.append(w)
        out.append(oh)
        wts.append(wh)
    return out, wts
