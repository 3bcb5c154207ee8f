"""float64 oracle for the memory-linear ("Flash") attention path's row statistics and
its backward pass.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports or calls anything
here, and nothing here imports the HIP library.

Riftco's "Two exact full-sequence algorithms" section: the Flash path saves per-row
softmax statistics of shape [B, H, T] instead of the [B, H, T, T] probabilities, and
its backward pass recomputes every needed probability from Q, K and those statistics,
then applies the same exact softmax vector-Jacobian product as the materialized path;
a context upstream gradient produces query, key and value gradients.  The page saves
the row maximum and the exponential sum; one number carries the same information, the
log-sum-exp of the row, lse_i = log sum_j exp(s_ij), from which P_ij = exp(s_ij - lse_i).

This module writes the definitions out with materialized probabilities (small shapes
only), in the notation of the attention oracle (scores s = scale * Q K^T, causal -inf
mask, query head h reads K/V head h // (Hq / Hkv)):

    P      = softmax_j(s)
    dV     = P^T dO                    summed over the query heads of each K/V head
    dP     = dO V^T
    dS     = P * (dP - sum_j P * dP)   the softmax vector-Jacobian product, row by row
    dQ     = scale * dS K
    dK     = scale * dS^T Q            summed over the query heads of each K/V head
"""
from __future__ import annotations

import numpy as np


def _scores(q, k, scale, causal):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    G = q.shape[1] // k.shape[1]
    ke = np.repeat(k, G, axis=1)
    s = np.matmul(q, np.swapaxes(ke, -1, -2)) * scale
    if causal:
        T, Tk = q.shape[2], k.shape[2]
        if T != Tk:
            raise ValueError("full-sequence attention: q and k have the same length")
        s = np.where(np.arange(Tk)[None, :] > np.arange(T)[:, None], -np.inf, s)
    return s, G


def lse(q, k, scale, causal=True):
    """Row log-sum-exp of the (masked) scores: [B, Hq, T], natural log."""
    s, _ = _scores(q, k, scale, causal)
    m = s.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(s - m).sum(axis=-1, keepdims=True)))[..., 0]


def probs(q, k, scale, causal=True):
    s, _ = _scores(q, k, scale, causal)
    m = s.max(axis=-1, keepdims=True)
    w = np.exp(s - m)
    return w / w.sum(axis=-1, keepdims=True)


def backward(q, k, v, dout, scale, causal=True):
    """Gradients of <dout, attention(q, k, v)>: dq [B,Hq,T,d], dk and dv [B,Hkv,T,d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(dout, dtype=np.float64)
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    P = probs(q, k, scale, causal)                       # [B, Hq, T, T]
    ke = np.repeat(k, G, axis=1)
    ve = np.repeat(v, G, axis=1)
    dv_e = np.matmul(np.swapaxes(P, -1, -2), do)         # [B, Hq, T, d]
    dP = np.matmul(do, np.swapaxes(ve, -1, -2))          # [B, Hq, T, T]
    dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
    dq = scale * np.matmul(dS, ke)
    dk_e = scale * np.matmul(np.swapaxes(dS, -1, -2), q)
    # the chain rule through repeat_interleave: a K/V head's gradient is the sum over
    # the query heads that read it
    dk = dk_e.reshape(B, Hkv, G, T, d).sum(axis=2)
    dv = dv_e.reshape(B, Hkv, G, T, d).sum(axis=2)
    return dq, dk, dv
