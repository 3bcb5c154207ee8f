"""float64 oracle for the step before cached decode: KV-cache append with NeoX RoPE on K.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports or calls
anything here, and nothing here imports the HIP library.

What it computes (Hesper's attention layer, "fusedRopeKAndCacheWriteKernel" and
its batched prefill companion; the forge chapter's ``apply_rope(..., offset=start_pos)``
followed by the cache append):

* new token i of sequence b sits at absolute position ``p = start_pos + i``;
* its K row is rotated by NeoX RoPE at position p: head dims j and j + d/2 form a
  rotation pair (the pages: "the pair partner is at dim + halfDim"), turned by the
  angle ``p * base**(-2j/d) / freq_factors[j]`` (freq_factors default to 1);
* the rotated K row and the plain V row are written to cache row p of their K/V
  head; every other cache row keeps its value.

The pages name NeoX RoPE, ``ropeBase`` and a ``freq_factors`` input but their
equations are not rendered; the rotation written out here is the plain reading
(RoFormer's rotary embedding in the rotate-half pairing, the angle divided by the
per-pair factor).  Everything is float64; rounding to the cache dtype is left to
the comparison.
"""
from __future__ import annotations

import numpy as np


def rope_angles(positions, d: int, base: float, freq_factors=None):
    """Angle of rotation pair j at each absolute position: [len(positions), d/2]."""
    if d % 2:
        raise ValueError("NeoX RoPE pairs dims j and j + d/2: d must be even")
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    inv_freq = np.power(float(base), -2.0 * j / d)
    if freq_factors is not None:
        ff = np.asarray(freq_factors, dtype=np.float64)
        if ff.shape != (half,):
            raise ValueError("freq_factors must hold d/2 values")
        inv_freq = inv_freq / ff
    return np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]


def rope_neox(x, positions, base: float, freq_factors=None):
    """Rotate the last axis of x [..., T, d] at the absolute positions [T]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = rope_angles(positions, d, base, freq_factors)  # [T, half]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def kv_append(kcache, vcache, k_new, v_new, start_pos: int, rope_base: float = 0.0,
              freq_factors=None):
    """Caches [B, Hkv, L, d] after writing the new tokens [B, n, Hkv, d] at start_pos.

    rope_base > 0 rotates K (NeoX RoPE at each token's absolute position); 0 writes
    K unrotated.  Returns float64 copies; the inputs are not modified.
    """
    kc = np.array(kcache, dtype=np.float64)
    vc = np.array(vcache, dtype=np.float64)
    kn = np.asarray(k_new, dtype=np.float64)
    vn = np.asarray(v_new, dtype=np.float64)
    B, Hkv, L, d = kc.shape
    n = kn.shape[1]
    if kn.shape != (B, n, Hkv, d) or vn.shape != kn.shape or vc.shape != kc.shape:
        raise ValueError("shape mismatch")
    if start_pos < 0 or start_pos + n > L:
        raise ValueError("the new tokens must fit in the cache")
    pos = start_pos + np.arange(n)
    kh = np.swapaxes(kn, 1, 2)  # [B, Hkv, n, d]
    if rope_base > 0:
        kh = rope_neox(kh, pos, rope_base, freq_factors)
    kc[:, :, start_pos:start_pos + n, :] = kh
    vc[:, :, start_pos:start_pos + n, :] = np.swapaxes(vn, 1, 2)
    return kc, vc


def kv_append_paged(kpool, vpool, block_table, seq_lens, k_new, v_new, rope_base: float = 0.0,
                    freq_factors=None):
    """Paged pools [num_blocks, Hkv, bs, d] after writing the new tokens of each sequence.

    The new tokens of sequence b are its last n positions, seq_lens[b] - n + i; position
    p lives in block block_table[b][p // bs], row p % bs.
    """
    kp = np.array(kpool, dtype=np.float64)
    vp = np.array(vpool, dtype=np.float64)
    kn = np.asarray(k_new, dtype=np.float64)
    vn = np.asarray(v_new, dtype=np.float64)
    nblk, Hkv, bs, d = kp.shape
    B, n = kn.shape[:2]
    table = np.asarray(block_table)
    for b in range(B):
        L = int(seq_lens[b])
        if L < n or (L + bs - 1) // bs > table.shape[1]:
            raise ValueError("sequence %d: length does not fit its table" % b)
        pos = np.arange(L - n, L)
        kh = np.swapaxes(kn[b], 0, 1)  # [Hkv, n, d]
        if rope_base > 0:
            kh = rope_neox(kh, pos, rope_base, freq_factors)
        for i, p in enumerate(pos):
            blk = int(table[b, p // bs])
            if not 0 <= blk < nblk:
                raise ValueError("table entry outside the pool")
            kp[blk, :, p % bs, :] = kh[:, i, :]
            vp[blk, :, p % bs, :] = vn[b, i]
    return kp, vp
