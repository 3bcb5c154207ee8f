"""float64 CPU oracle for causal grouped-query attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP library never imports, links or
calls anything here, and nothing here imports the HIP library.

Two independent implementations of one definition live in this package:

* ``gqa_oracle.c`` (loaded here through ctypes): per-row materialized scores,
  libm ``exp`` in float64, threads over independent (batch, head) units.
* ``ref_numpy.py``: the same definition as whole-matrix NumPy float64 algebra.

The definition (scores = scale * Q K^T, additive -inf causal mask, softmax over
keys, times V; query head h reads K/V head h // (Hq // Hkv)) follows Riftco's
"Causal Multi-Head Self-Attention" page ("Dataflow and shapes", "The causal
mask"), the "Grouped-Query Attention" chapter (sections 5.1 and 5.2) and, for
cached decode, makarna's ``CausalAttentionCached``: the new tokens sit at
absolute positions startPos .. startPos+newTokens-1, each sees every cached key
up to and including its own position, and the scale is 1/sqrt(headDim).
Paged decode (makarna's ``CausalAttentionPackedBlocks``) is that same cached
decode over the history assembled from the blocks a block table names.  The
views form (makarna's ``CausalAttentionBlocks``) is written out on its own terms
in ``decode_views``: a list of token-major views, each holding the keys at
positions Start .. Start+Length-1, of which new token i sees those below
startPos+i+1.

Inputs are widened exactly to float64 (bf16 and fp32 values are all exactly
representable), so the oracle never rounds an input.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gqa_oracle.c into liboracle.so with the host C compiler.

    No -ffast-math: the oracle keeps IEEE float64 semantics.
    """
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-D_POSIX_C_SOURCE=200809L", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_attention.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_attention.argtypes = [dp, dp, dp, dp, dp,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                         ctypes.c_long, ctypes.c_long, ctypes.c_int]
        lib.oracle_default_threads.restype = ctypes.c_int
        lib.oracle_default_threads.argtypes = []
        _lib = lib
    return _lib


def to_f64(x) -> np.ndarray:
    """Exact widening of a numpy array or torch tensor (fp32 / bf16 / fp64) to float64."""
    if hasattr(x, "detach"):  # torch tensor: widen through torch, which is exact for bf16/fp32
        import torch

        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    return int(_load().oracle_default_threads())


def attention(q, k, v, scale: float, causal: bool = True, pos0: int = 0,
              nthreads: int = 0, want_probs: bool = False, window: int = 0):
    """Materialized float64 attention in head-major layout.

    q: [B, Hq, Tq, d]; k, v: [B, Hkv, Tk, d].  Query row i is at absolute
    position pos0 + i.  window >= 1 (causal only) keeps keys pos0+i-window+1 ..
    pos0+i; 0 means no window.  Returns out [B, Hq, Tq, d] (float64), and P
    [B, Hq, Tq, Tk] as well when want_probs.
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if v.shape != k.shape or Bk != B or dk != d:
        raise ValueError("shape mismatch: q %s k %s v %s" % (q.shape, k.shape, v.shape))
    out = np.zeros((B, Hq, Tq, d), dtype=np.float64)
    probs = np.zeros((B, Hq, Tq, Tk), dtype=np.float64) if want_probs else None
    rc = _load().oracle_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(probs),
                                  B, Hq, Hkv, Tq, Tk, d, float(scale), int(bool(causal)),
                                  int(pos0), int(window), int(nthreads))
    if rc != 0:
        raise ValueError("oracle_attention rejected its arguments (rc=%d)" % rc)
    return (out, probs) if want_probs else out


def prefill(q, k, v, scale: float, causal: bool = True, nthreads: int = 0, window: int = 0):
    """Full-sequence prefill: q [B,Hq,T,d], k/v [B,Hkv,T,d] -> out [B,Hq,T,d].
    window >= 1: local causal attention over the last `window` positions."""
    return attention(q, k, v, scale, causal, 0, nthreads, window=window)


def decode_cached(q, kcache, vcache, start_pos: int, nthreads: int = 0, window: int = 0):
    """Cached decode: q [B,n,Hq,d] (new tokens, token-major like makarna's Q),
    kcache/vcache [B,Hkv,totalLen,d] already holding the new tokens at
    start_pos..start_pos+n-1.  Scale is 1/sqrt(d) as in CausalAttentionCached.
    window >= 1: token i sees keys start_pos+i-window+1 .. start_pos+i only.
    Returns out [B,n,Hq,d] (float64).
    """
    qh = to_f64(q).transpose(0, 2, 1, 3)  # layout change only: [B,Hq,n,d]
    d = qh.shape[-1]
    out = attention(qh, kcache, vcache, 1.0 / math.sqrt(d), True, start_pos, nthreads,
                    window=window)
    return np.ascontiguousarray(out.transpose(0, 2, 1, 3))


def gather_paged(pool, block_table, seq_len: int, block_size: int, b: int):
    """The logical K (or V) history of sequence b out of a block pool.

    pool: [num_blocks, Hkv, block_size, d], head-major inside each block (makarna's
    packed view layout [kvHead][tokenWithinBlock][headDim]).  Logical block i of the
    sequence is the view with Start = i * block_size and Length = min(block_size,
    seq_len - Start); its physical block is block_table[b][i].  Table entries past the
    last block the sequence needs are never read.  Returns [Hkv, seq_len, d] (float64).
    """
    pool = to_f64(pool)
    nb, hkv, bs, d = pool.shape
    if bs != block_size:
        raise ValueError("pool block size %d != block_size %d" % (bs, block_size))
    nblk = -(-seq_len // block_size)
    table = np.asarray(block_table)
    if nblk > table.shape[1]:
        raise ValueError("sequence %d needs %d blocks, table has %d" % (b, nblk, table.shape[1]))
    ids = [int(x) for x in table[b, :nblk]]
    if any(i < 0 or i >= nb for i in ids):
        raise ValueError("sequence %d: block id out of range" % b)
    hist = np.empty((hkv, nblk * block_size, d), dtype=np.float64)
    for i, blk in enumerate(ids):  # view i covers positions i*bs .. i*bs+bs-1
        hist[:, i * block_size:(i + 1) * block_size, :] = pool[blk]
    return hist[:, :seq_len, :]


def decode_paged(q, kpool, vpool, block_table, seq_lens, block_size: int, nthreads: int = 0,
                 window: int = 0):
    """Paged (block-table) cached decode: the cached decode of every sequence b over
    the history gather_paged assembles, with its own length seq_lens[b] (new tokens
    at seq_lens[b]-n .. seq_lens[b]-1).  q [B,n,Hq,d] -> out [B,n,Hq,d] (float64).
    This is makarna's CausalAttentionPackedBlocks with one view per table entry.
    """
    q = to_f64(q)
    B, n, Hq, d = q.shape
    out = np.zeros((B, n, Hq, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L < n:
            raise ValueError("sequence %d: length %d < newTokens %d" % (b, L, n))
        if n == 0:
            continue
        kh = gather_paged(kpool, block_table, L, block_size, b)
        vh = gather_paged(vpool, block_table, L, block_size, b)
        out[b] = decode_cached(q[b:b + 1], kh[None], vh[None], L - n, nthreads, window)[0]
    return out


def decode_views(q, views, start_pos: int, n_kv_heads: int):
    """makarna's CausalAttentionBlocks for one sequence, materialized in float64.

    q: [n, Hq, d] new-token queries (token-major).  views: iterable of (start, K, V),
    K and V [length, Hkv*d] token-major (all KV heads of a position side by side),
    holding the keys at absolute positions start .. start+length-1.  New token i sits
    at start_pos+i and sees every key of every view whose position is below
    start_pos+i+1; the views are taken in order of start (their order in the list
    does not matter) and a view of length 0 holds nothing.  Query head h reads KV
    head h // (Hq // Hkv); the scale is 1/sqrt(d).  A token that sees no key gets a
    zero row, as the page's loop leaves it.  Returns [n, Hq, d] (float64).
    """
    q = to_f64(q)
    n, Hq, d = q.shape
    if Hq % n_kv_heads:
        raise ValueError("Hq %d is not a multiple of Hkv %d" % (Hq, n_kv_heads))
    group = Hq // n_kv_heads
    vs = []
    for start, kv_k, kv_v in views:
        kv_k, kv_v = to_f64(kv_k), to_f64(kv_v)
        if kv_k.shape != kv_v.shape or kv_k.ndim != 2 or kv_k.shape[1] != n_kv_heads * d:
            raise ValueError("a view's K and V must both be [length, Hkv*d]")
        if kv_k.shape[0] > 0:
            vs.append((int(start), kv_k.reshape(-1, n_kv_heads, d), kv_v.reshape(-1, n_kv_heads, d)))
    vs.sort(key=lambda t: t[0])
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((n, Hq, d), dtype=np.float64)
    for i in range(n):
        limit = start_pos + i + 1  # keys at positions < limit are visible
        ks, vv = [], []
        for start, vk, vval in vs:
            if start >= limit:
                continue
            m = min(vk.shape[0], limit - start)
            ks.append(vk[:m])
            vv.append(vval[:m])
        if not ks:
            continue
        kc, vc = np.concatenate(ks), np.concatenate(vv)  # [keys, Hkv, d]
        for h in range(Hq):
            s_ = (kc[:, h // group, :] @ q[i, h]) * scale
            w = np.exp(s_ - s_.max())
            out[i, h] = (w / w.sum()) @ vc[:, h // group, :]
    return out


def views_from_blocks(kpool, vpool, block_table, seq_len: int, block_size: int, b: int):
    """The views of sequence b out of token-major block pools [num_blocks, block_size,
    Hkv, d]: logical block i is the view with Start = i*block_size and Length =
    min(block_size, seq_len - Start), its K and V the first Length rows of physical
    block block_table[b][i], each row [Hkv*d]."""
    kpool, vpool = to_f64(kpool), to_f64(vpool)
    nb, bs, hkv, d = kpool.shape
    if bs != block_size or vpool.shape != kpool.shape:
        raise ValueError("pools must be [num_blocks, %d, Hkv, d]" % block_size)
    table = np.asarray(block_table)
    views = []
    for i in range(-(-seq_len // block_size)):
        blk = int(table[b, i])
        if blk < 0 or blk >= nb:
            raise ValueError("sequence %d: block id out of range" % b)
        length = min(block_size, seq_len - i * block_size)
        views.append((i * block_size, kpool[blk, :length].reshape(length, hkv * d),
                      vpool[blk, :length].reshape(length, hkv * d)))
    return views


def decode_blocks(q, kpool, vpool, block_table, seq_lens, block_size: int):
    """Cached decode over token-major blocks: decode_views of every sequence b over the
    views of its table row, with its new tokens at seq_lens[b]-n .. seq_lens[b]-1.
    q [B,n,Hq,d] -> out [B,n,Hq,d] (float64)."""
    q = to_f64(q)
    B, n, Hq, d = q.shape
    hkv = int(kpool.shape[2])
    out = np.zeros((B, n, Hq, d), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        if L < n:
            raise ValueError("sequence %d: length %d < newTokens %d" % (b, L, n))
        if n == 0:
            continue
        views = views_from_blocks(kpool, vpool, block_table, L, block_size, b)
        out[b] = decode_views(q[b], views, L - n, hkv)
    return out


def probs(q, k, v, scale: float, causal: bool = True, pos0: int = 0, window: int = 0):
    """The probability matrix P [B,Hq,Tq,Tk] (small shapes only)."""
    return attention(q, k, v, scale, causal, pos0, 1, want_probs=True, window=window)[1]
