"""Gradients of ALiBi attention in plain fp64 (test infrastructure, not the product).

The pages define the forward only: out = softmax(Q K^T / sqrt(d) + B) V with
the fixed ALiBi bias B = -m (i - j) and the causal mask ("When Attention Goes
Blind", Sec. 3.1 Eq. 1-3; the slopes are fixed, not learned: abhik.ai,
"Different heads, different distance penalties"). Sec. 4.2 / 5.1 of the
paper train such models and discuss what underflow does to the backward
pass, which is the reason the gradients are on the hot path here.

The gradients below are the chain rule of that definition, step by step:
  P = softmax(logits), O = P V
  dV = P^T dO
  dP = dO V^T
  dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian applied row by row)
  dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
The bias is a constant, so it has no gradient of its own. The row log-sum-exp
of the logits (natural log) is what a forward pass keeps for this backward.

The paper trains its models with the Sec. 3.4 mitigations too. Two of them
change only that constant bias and therefore only the logits here: the clamp,
B* = max(B, c_clamp), and the log-scaled distance, B = -m log(D + 1) (the
definitions of oracle.mitigations, with D = i - j under the mask and |i - j|
without it). The third, the soft cap A* = z tanh(A / z) of the content logit
A = q k / sqrt(d), sits between the scores and the logits, so one more factor
of the chain rule appears: dlogit/dA = 1 - tanh(A / z)^2, applied to dS before
dQ and dK are formed.
"""
from __future__ import annotations

import math

import numpy as np

from .alibi_ref import _f64, bias_ref, distance_ref, softmax_rows_ref


def _logits(q, k, m, causal, clamp=None, log_distance=False, softcap=None):
    a = (q @ k.T) / math.sqrt(q.shape[-1])
    if softcap is not None:
        a = float(softcap) * np.tanh(a / float(softcap))
    dist = distance_ref(q.shape[0], k.shape[0])
    if clamp is None and not log_distance:
        bias = bias_ref(m, dist, causal)
    else:
        dd = np.abs(dist).astype(np.float64)
        if log_distance:
            dd = np.log(dd + 1.0)
        bias = -float(m) * dd
        if clamp is not None:
            bias = np.maximum(bias, float(clamp))
    logits = a + bias
    if causal:
        logits = np.where(dist < 0, -np.inf, logits)
    return logits


def lse_head_ref(q, k, m, causal=True, clamp=None, log_distance=False, softcap=None):
    """Row log-sum-exp (natural log) of one head's logits, fp64."""
    logits = _logits(_f64(q), _f64(k), m, causal, clamp, log_distance, softcap)
    mx = np.max(logits, axis=-1, keepdims=True)
    return (mx + np.log(np.sum(np.exp(logits - mx), axis=-1, keepdims=True)))[:, 0]


def attn_backward_head_ref(q, k, v, do, m, causal=True, magnitudes=False, clamp=None, log_distance=False,
                           softcap=None):
    """(dq, dk, dv) of one head for the upstream gradient do, fp64; clamp,
    log_distance and softcap as in oracle.mitigations (a bias floor, ln(D + 1)
    distances, the content logit capped at z tanh(A / z)).

    With ``magnitudes`` also the sums of absolute products behind each gradient
    element, (|dS| |K| / sqrt(d), |dS|^T |Q| / sqrt(d), P^T |dO|): the scale of
    its terms, against which cancellation among them is measured (each bounds
    the absolute value of its gradient).
    """
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p = softmax_rows_ref(_logits(q, k, m, causal, clamp, log_distance, softcap))
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
    scale = 1.0 / math.sqrt(q.shape[-1])
    if softcap is not None:
        # the logit's derivative with respect to the content logit A
        th = np.tanh((q @ k.T) * scale / float(softcap))
        ds = ds * (1.0 - th * th)
    grads = (ds @ k * scale, ds.T @ q * scale, dv)
    if not magnitudes:
        return grads
    a = np.abs(ds)
    return grads, (a @ np.abs(k) * scale, a.T @ np.abs(q) * scale, p.T @ np.abs(do))


def attn_backward_ref(q, k, v, do, slopes, causal=True, clamp=None, log_distance=False, softcap=None):
    """Multi-head gradients: inputs (B, H, N, d); returns dq, dk, dv (B, H, N, d) fp64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    slopes = np.asarray(_f64(slopes)).reshape(-1)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            dq[b, h], dk[b, h], dv[b, h] = attn_backward_head_ref(q[b, h], k[b, h], v[b, h], do[b, h],
                                                                  slopes[h], causal, clamp=clamp,
                                                                  log_distance=log_distance, softcap=softcap)
    return dq, dk, dv


def lse_ref(q, k, slopes, causal=True, clamp=None, log_distance=False, softcap=None):
    """Row log-sum-exp (natural log), (B, H, N) fp64."""
    q, k = _f64(q), _f64(k)
    slopes = np.asarray(_f64(slopes)).reshape(-1)
    out = np.empty(q.shape[:3], dtype=np.float64)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out[b, h] = lse_head_ref(q[b, h], k[b, h], slopes[h], causal, clamp, log_distance, softcap)
    return out
