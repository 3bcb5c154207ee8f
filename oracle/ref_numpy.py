"""Second, independent float64 oracle in NumPy (TEST INFRASTRUCTURE ONLY).

It restates the same definition as the C oracle with whole-matrix algebra, the
way the "Grouped-Query Attention" chapter's eager reference does it (section
5.2, "The read itself"): expand K/V heads with repeat-interleave semantics,
form the full score grid, add the causal -inf bias (and, for local attention,
-inf below the window), softmax over keys, multiply by V.  Section 5.3 of that chapter checks one implementation against an
independent second one; this module plays that role for the C oracle.
Only meant for small shapes (it materializes [B, Hq, Tq, Tk]) and finite inputs
(a non-finite future value would reach earlier rows through 0 * inf here).
"""
from __future__ import annotations

import numpy as np


def attention(q, k, v, scale, causal=True, pos0=0, return_probs=False, window=0):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    # np.repeat along the head axis = repeat_interleave: head h reads kv head h // G
    ke = np.repeat(k, G, axis=1)
    ve = np.repeat(v, G, axis=1)
    s = np.matmul(q, np.swapaxes(ke, -1, -2)) * scale  # [B,Hq,Tq,Tk]
    Tk = k.shape[2]
    if window and not causal:
        raise ValueError("a local window needs the causal mask")
    if causal:
        pos = pos0 + np.arange(Tq)[:, None]
        keys = np.arange(Tk)[None, :]
        bias = np.where(keys > pos, -np.inf, 0.0)
        if window:  # local attention: only the last `window` positions up to the query's own
            bias = np.where(keys < pos - window + 1, -np.inf, bias)
        s = s + bias
    s = s - s.max(axis=-1, keepdims=True)
    w = np.exp(s)
    p = w / w.sum(axis=-1, keepdims=True)
    out = np.matmul(p, ve)
    return (out, p) if return_probs else out
