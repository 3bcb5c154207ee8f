"""Thin Python binding of libgqa_attn.so (causal grouped-query attention on gfx950).

The functions mirror the C ABI in include/gqa_attn.h one for one and only marshal
arguments: they check torch tensors' device, dtype, shape and contiguity, pass raw
device pointers and the current HIP stream, and turn a negative status into an
exception.  Every step of the computation runs in the library's HIP kernels; there
is no fallback.  Importing this package fails if the library has not been built
(``python grouped_query_attention_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgqa_attn.so")

GQA_F32, GQA_BF16 = 0, 1
GQA_OK, GQA_EINVAL, GQA_EUNSUPPORTED, GQA_EWORKSPACE, GQA_EHIP, GQA_ESCRATCH = 0, -1, -2, -3, -4, -5
GQA_NOALLOC_SCRATCH_BYTES = 64 << 20  # the fixed scratch of attn_decode_cached_noalloc
GQA_ALGO_AUTO, GQA_ALGO_GENERIC, GQA_ALGO_MFMA, GQA_ALGO_MFMA_SPLIT = 0, 1, 2, 3

# every symbol include/gqa_attn.h declares
EXPORTED = ("attn_prefill", "attn_prefill_ex", "attn_prefill_window", "attn_decode_workspace_bytes",
            "attn_decode_num_splits", "attn_decode_cached", "attn_decode_window_workspace_bytes",
            "attn_decode_window", "attn_decode_paged_workspace_bytes", "attn_decode_paged",
            "attn_decode_paged_window_workspace_bytes", "attn_decode_paged_window", "attn_decode_blocks",
            "attn_kv_append",
            "attn_kv_append_paged", "attn_prefill_lse", "attn_backward_workspace_bytes", "attn_backward",
            "attn_strerror", "attn_decode_cached_noalloc")

if not os.path.exists(LIB_PATH):
    raise ImportError("libgqa_attn.so is not built (%s); run python grouped_query_attention_amd/build.py"
                      % LIB_PATH)

lib = ctypes.CDLL(LIB_PATH)
_i, _vp, _f, _sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
lib.attn_prefill.restype = _i
lib.attn_prefill.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
lib.attn_prefill_ex.restype = _i
lib.attn_prefill_ex.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp]
lib.attn_decode_workspace_bytes.restype = _sz
lib.attn_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
lib.attn_decode_num_splits.restype = _i
lib.attn_decode_num_splits.argtypes = [_i, _i, _i, _i, _i, _i, _i]
lib.attn_decode_cached.restype = _i
lib.attn_decode_cached.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
lib.attn_decode_paged_workspace_bytes.restype = _sz
lib.attn_decode_paged_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
lib.attn_decode_paged.restype = _i
lib.attn_decode_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                  _vp, _sz, _vp]
lib.attn_prefill_window.restype = _i
lib.attn_prefill_window.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
lib.attn_decode_window_workspace_bytes.restype = _sz
lib.attn_decode_window_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
lib.attn_decode_window.restype = _i
lib.attn_decode_window.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
lib.attn_decode_paged_window_workspace_bytes.restype = _sz
lib.attn_decode_paged_window_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i, _i]
lib.attn_decode_paged_window.restype = _i
lib.attn_decode_paged_window.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                                         _i, _i, _vp, _sz, _vp]
lib.attn_decode_blocks.restype = _i
lib.attn_decode_blocks.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _i,
                                   _vp, _sz, _vp]
lib.attn_kv_append.restype = _i
lib.attn_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _vp]
lib.attn_kv_append_paged.restype = _i
lib.attn_kv_append_paged.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                                     _i, _vp]
lib.attn_prefill_lse.restype = _i
lib.attn_prefill_lse.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
lib.attn_backward_workspace_bytes.restype = _sz
lib.attn_backward_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
lib.attn_backward.restype = _i
lib.attn_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i,
                              _vp, _sz, _vp]
lib.attn_decode_cached_noalloc.restype = _i
lib.attn_decode_cached_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]
lib.attn_strerror.restype = ctypes.c_char_p
lib.attn_strerror.argtypes = [_i]


class GQAError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__("%s: %s (status %d)" % (what, attn_strerror(code), code))


def attn_strerror(code: int) -> str:
    return lib.attn_strerror(int(code)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GQA_F32
    if t.dtype == torch.bfloat16:
        return GQA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _dev_ptr(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr() if t.numel() else None


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _empty(shape, dtype, device, stream):
    """A new tensor for the library to write on `stream`.  It is allocated with that
    stream current, so torch's caching allocator hands its block out again only in that
    stream's order: a workspace dropped on return, or an output the caller frees, is
    never reused by another stream while the kernels may still write it."""
    if stream is None:
        return torch.empty(shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(shape, dtype=dtype, device=device)


def attn_prefill(q, k, v, scale=None, causal=True, out=None, algo=GQA_ALGO_AUTO, stream=None,
                 window=None):
    """Causal (or full) GQA prefill.  q [B,Hq,T,d]; k, v [B,Hkv,T,d] (same dtype,
    float32 or bfloat16).  Returns out [B,Hq,T,d] float32 (written into `out` if given).
    window=W (causal only) calls attn_prefill_window: row i sees keys i-W+1 .. i."""
    B, Hq, T, d = q.shape
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != T or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, Hkv, T, d] matching q %s; got %s %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    Hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = _empty((B, Hq, T, d), torch.float32, q.device, stream)
    elif out.shape != q.shape or out.dtype != torch.float32:
        raise ValueError("out must be float32 of shape %s" % (tuple(q.shape),))
    if window is not None:
        if not causal or algo != GQA_ALGO_AUTO:
            raise ValueError("a local window needs causal=True and the automatic kernel choice")
        rc = lib.attn_prefill_window(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                                     _dev_ptr(out, "out"), B, Hq, Hkv, T, d, float(scale), int(window),
                                     _dtype_code(q), _stream_handle(stream, q.device))
        if rc != GQA_OK:
            raise GQAError(rc, "attn_prefill_window")
        return out
    rc = lib.attn_prefill_ex(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                             B, Hq, Hkv, T, d, float(scale), int(bool(causal)), _dtype_code(q), int(algo),
                             _stream_handle(stream, q.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_prefill")
    return out


def attn_decode_workspace_bytes(B, new_tokens, total_len, Hq, Hkv, d, dtype=GQA_BF16) -> int:
    return int(lib.attn_decode_workspace_bytes(B, new_tokens, total_len, Hq, Hkv, d, int(dtype)))


def attn_decode_num_splits(B, new_tokens, total_len, Hq, Hkv, d, dtype=GQA_BF16) -> int:
    return int(lib.attn_decode_num_splits(B, new_tokens, total_len, Hq, Hkv, d, int(dtype)))


def attn_decode_window_workspace_bytes(B, new_tokens, total_len, Hq, Hkv, d, window,
                                       dtype=GQA_BF16) -> int:
    return int(lib.attn_decode_window_workspace_bytes(B, new_tokens, total_len, Hq, Hkv, d, int(window),
                                                      int(dtype)))


def attn_decode_cached(q, kcache, vcache, start_pos, out=None, workspace=None, stream=None, window=None):
    """Cached decode.  q [B,n,Hq,d] (new tokens, token-major); kcache, vcache
    [B,Hkv,L,d] holding positions 0..L-1 with the new tokens at start_pos..start_pos+n-1.
    Scale is 1/sqrt(d).  Returns out [B,n,Hq,d] float32.  A workspace tensor of at least
    attn_decode_workspace_bytes(...) bytes is allocated here when not supplied.  window=W
    keeps new token i's keys start_pos+i-W+1 .. start_pos+i only (attn_decode_window)."""
    B, n, Hq, d = q.shape
    if kcache.dim() != 4 or kcache.shape[0] != B or kcache.shape[3] != d or vcache.shape != kcache.shape:
        raise ValueError("kcache, vcache must be [B, Hkv, L, d]; got %s %s"
                         % (tuple(kcache.shape), tuple(vcache.shape)))
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise TypeError("q, kcache, vcache must share one dtype")
    Hkv, L = kcache.shape[1], kcache.shape[2]
    dt = _dtype_code(q)
    if out is None:
        out = _empty((B, n, Hq, d), torch.float32, q.device, stream)
    elif out.shape != q.shape or out.dtype != torch.float32:
        raise ValueError("out must be float32 of shape %s" % (tuple(q.shape),))
    if window is None:
        need = attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, dt)
    else:
        need = attn_decode_window_workspace_bytes(B, n, L, Hq, Hkv, d, window, dt)
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if window is None:
        rc = lib.attn_decode_cached(_dev_ptr(q, "q"), _dev_ptr(kcache, "kcache"), _dev_ptr(vcache, "vcache"),
                                    _dev_ptr(out, "out"), n, L, int(start_pos), Hq, Hkv, d, B, dt,
                                    ws_ptr, ws_bytes, _stream_handle(stream, q.device))
        what = "attn_decode_cached"
    else:
        rc = lib.attn_decode_window(_dev_ptr(q, "q"), _dev_ptr(kcache, "kcache"), _dev_ptr(vcache, "vcache"),
                                    _dev_ptr(out, "out"), n, L, int(start_pos), Hq, Hkv, d, B, int(window),
                                    dt, ws_ptr, ws_bytes, _stream_handle(stream, q.device))
        what = "attn_decode_window"
    if rc != GQA_OK:
        raise GQAError(rc, what)
    return out


def attn_decode_cached_noalloc(q, kcache, vcache, start_pos, out, stream=None):
    """attn_decode_cached without a workspace: the library keeps the split-KV partials in
    its fixed device scratch (GQA_NOALLOC_SCRATCH_BYTES per GPU), so the call allocates
    nothing.  out [B,n,Hq,d] float32 must be supplied.  Calls that overlap on one GPU
    share the scratch and race; shapes needing more scratch raise GQAError with
    GQA_ESCRATCH."""
    B, n, Hq, d = q.shape
    if kcache.dim() != 4 or kcache.shape[0] != B or kcache.shape[3] != d or vcache.shape != kcache.shape:
        raise ValueError("kcache, vcache must be [B, Hkv, L, d]; got %s %s"
                         % (tuple(kcache.shape), tuple(vcache.shape)))
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise TypeError("q, kcache, vcache must share one dtype")
    if out is None or out.shape != q.shape or out.dtype != torch.float32:
        raise ValueError("out must be float32 of shape %s" % (tuple(q.shape),))
    Hkv, L = kcache.shape[1], kcache.shape[2]
    rc = lib.attn_decode_cached_noalloc(_dev_ptr(q, "q"), _dev_ptr(kcache, "kcache"), _dev_ptr(vcache, "vcache"),
                                        _dev_ptr(out, "out"), n, L, int(start_pos), Hq, Hkv, d, B,
                                        _dtype_code(q), _stream_handle(stream, q.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_decode_cached_noalloc")
    return out


def attn_decode_paged_workspace_bytes(B, new_tokens, Hq, Hkv, d, block_size, max_blocks,
                                      dtype=GQA_BF16) -> int:
    return int(lib.attn_decode_paged_workspace_bytes(B, new_tokens, Hq, Hkv, d, block_size,
                                                     max_blocks, int(dtype)))


def attn_decode_paged_window_workspace_bytes(B, new_tokens, Hq, Hkv, d, block_size, max_blocks, window,
                                             dtype=GQA_BF16) -> int:
    return int(lib.attn_decode_paged_window_workspace_bytes(B, new_tokens, Hq, Hkv, d, block_size,
                                                            max_blocks, int(window), int(dtype)))


def attn_decode_paged(q, kpool, vpool, block_table, seq_lens, out=None, workspace=None,
                      stream=None, window=None):
    """Paged cached decode.  q [B,n,Hq,d] bf16; kpool, vpool [num_blocks,Hkv,block_size,d]
    bf16; block_table [B,max_blocks] int32 and seq_lens [B] int32 on the GPU (sequence b's
    history of seq_lens[b] positions, new tokens last, lives in the blocks its table row
    names in order).  Scale is 1/sqrt(d).  window=W keeps each new token's last W positions
    only (attn_decode_paged_window).  Returns out [B,n,Hq,d] float32."""
    B, n, Hq, d = q.shape
    if kpool.dim() != 4 or kpool.shape[3] != d or vpool.shape != kpool.shape:
        raise ValueError("kpool, vpool must be [num_blocks, Hkv, block_size, d]; got %s %s"
                         % (tuple(kpool.shape), tuple(vpool.shape)))
    if kpool.dtype != q.dtype or vpool.dtype != q.dtype:
        raise TypeError("q, kpool, vpool must share one dtype")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]; got %s %s"
                         % (tuple(block_table.shape), tuple(seq_lens.shape)))
    num_blocks, Hkv, bs = kpool.shape[0], kpool.shape[1], kpool.shape[2]
    max_blocks = block_table.shape[1]
    dt = _dtype_code(q)
    if out is None:
        out = _empty((B, n, Hq, d), torch.float32, q.device, stream)
    elif out.shape != q.shape or out.dtype != torch.float32:
        raise ValueError("out must be float32 of shape %s" % (tuple(q.shape),))
    if window is None:
        need = attn_decode_paged_workspace_bytes(B, n, Hq, Hkv, d, bs, max_blocks, dt)
    else:
        need = attn_decode_paged_window_workspace_bytes(B, n, Hq, Hkv, d, bs, max_blocks, window, dt)
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptrs = (_dev_ptr(q, "q"), _dev_ptr(kpool, "kpool"), _dev_ptr(vpool, "vpool"),
            _dev_ptr(block_table, "block_table"), _dev_ptr(seq_lens, "seq_lens"), _dev_ptr(out, "out"))
    if window is None:
        rc = lib.attn_decode_paged(*ptrs, B, n, Hq, Hkv, d, bs, max_blocks, num_blocks, dt,
                                   ws_ptr, ws_bytes, _stream_handle(stream, q.device))
        what = "attn_decode_paged"
    else:
        rc = lib.attn_decode_paged_window(*ptrs, B, n, Hq, Hkv, d, bs, max_blocks, num_blocks, int(window), dt,
                                          ws_ptr, ws_bytes, _stream_handle(stream, q.device))
        what = "attn_decode_paged_window"
    if rc != GQA_OK:
        raise GQAError(rc, what)
    return out


def attn_decode_blocks(q, kpool, vpool, block_table, seq_lens, out=None, workspace=None, stream=None):
    """Cached decode over token-major blocks (makarna's CausalAttentionBlocks views).
    q [B,n,Hq,d] bf16; kpool, vpool [num_blocks,block_size,Hkv,d] bf16; block_table
    [B,max_blocks] and seq_lens [B] int32 on the GPU, as in attn_decode_paged.  Scale is
    1/sqrt(d).  Returns out [B,n,Hq,d] float32."""
    B, n, Hq, d = q.shape
    if kpool.dim() != 4 or kpool.shape[3] != d or vpool.shape != kpool.shape:
        raise ValueError("kpool, vpool must be [num_blocks, block_size, Hkv, d]; got %s %s"
                         % (tuple(kpool.shape), tuple(vpool.shape)))
    if kpool.dtype != q.dtype or vpool.dtype != q.dtype:
        raise TypeError("q, kpool, vpool must share one dtype")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]; got %s %s"
                         % (tuple(block_table.shape), tuple(seq_lens.shape)))
    num_blocks, bs, Hkv = kpool.shape[0], kpool.shape[1], kpool.shape[2]
    max_blocks = block_table.shape[1]
    dt = _dtype_code(q)
    if out is None:
        out = _empty((B, n, Hq, d), torch.float32, q.device, stream)
    elif out.shape != q.shape or out.dtype != torch.float32:
        raise ValueError("out must be float32 of shape %s" % (tuple(q.shape),))
    need = attn_decode_paged_workspace_bytes(B, n, Hq, Hkv, d, bs, max_blocks, dt)
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.attn_decode_blocks(_dev_ptr(q, "q"), _dev_ptr(kpool, "kpool"), _dev_ptr(vpool, "vpool"),
                                _dev_ptr(block_table, "block_table"), _dev_ptr(seq_lens, "seq_lens"),
                                _dev_ptr(out, "out"), B, n, Hq, Hkv, d, bs, max_blocks, num_blocks, dt,
                                ws_ptr, ws_bytes, _stream_handle(stream, q.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_decode_blocks")
    return out


def _append_inputs(k_new, v_new, cache, freq_factors, rope_base):
    if k_new.dtype != torch.float32 or v_new.dtype != torch.float32:
        raise TypeError("k_new and v_new must be float32")
    if k_new.dim() != 4 or v_new.shape != k_new.shape:
        raise ValueError("k_new, v_new must be [B, newTokens, Hkv, d]; got %s %s"
                         % (tuple(k_new.shape), tuple(v_new.shape)))
    d = k_new.shape[3]
    ff = None
    if freq_factors is not None and rope_base:
        if freq_factors.dtype != torch.float32 or tuple(freq_factors.shape) != (d // 2,):
            raise ValueError("freq_factors must be float32 [d/2]")
        ff = _dev_ptr(freq_factors, "freq_factors")
    return ff, _dtype_code(cache)


def attn_kv_append(k_new, v_new, kcache, vcache, start_pos, rope_base=0.0, freq_factors=None,
                   stream=None):
    """Write the new tokens k_new, v_new [B,n,Hkv,d] float32 into kcache, vcache
    [B,Hkv,L,d] (float32 or bfloat16) at rows start_pos .. start_pos+n-1, rotating K with
    NeoX RoPE at each token's position when rope_base > 0 (attn_kv_append)."""
    B, n, Hkv, d = k_new.shape
    if kcache.dim() != 4 or vcache.shape != kcache.shape or kcache.dtype != vcache.dtype:
        raise ValueError("kcache, vcache must be [B, Hkv, L, d] of one dtype")
    if kcache.shape[0] != B or kcache.shape[1] != Hkv or kcache.shape[3] != d:
        raise ValueError("cache %s does not match new tokens %s" % (tuple(kcache.shape), tuple(k_new.shape)))
    ff, dt = _append_inputs(k_new, v_new, kcache, freq_factors, rope_base)
    rc = lib.attn_kv_append(_dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"), _dev_ptr(kcache, "kcache"),
                            _dev_ptr(vcache, "vcache"), ff, B, n, Hkv, d, kcache.shape[2], int(start_pos),
                            float(rope_base), dt, _stream_handle(stream, k_new.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_kv_append")


def attn_kv_append_paged(k_new, v_new, kpool, vpool, block_table, seq_lens, rope_base=0.0,
                         freq_factors=None, stream=None):
    """Paged append: the new tokens of sequence b are its last n positions of seq_lens[b],
    stored through block_table [B,max_blocks] int32 into kpool, vpool
    [num_blocks,Hkv,block_size,d] (attn_kv_append_paged)."""
    B, n, Hkv, d = k_new.shape
    if kpool.dim() != 4 or vpool.shape != kpool.shape or kpool.dtype != vpool.dtype:
        raise ValueError("kpool, vpool must be [num_blocks, Hkv, block_size, d] of one dtype")
    if kpool.shape[1] != Hkv or kpool.shape[3] != d:
        raise ValueError("pool %s does not match new tokens %s" % (tuple(kpool.shape), tuple(k_new.shape)))
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_blocks] and seq_lens [B]")
    ff, dt = _append_inputs(k_new, v_new, kpool, freq_factors, rope_base)
    rc = lib.attn_kv_append_paged(_dev_ptr(k_new, "k_new"), _dev_ptr(v_new, "v_new"), _dev_ptr(kpool, "kpool"),
                                  _dev_ptr(vpool, "vpool"), _dev_ptr(block_table, "block_table"),
                                  _dev_ptr(seq_lens, "seq_lens"), ff, B, n, Hkv, d, kpool.shape[2],
                                  block_table.shape[1], kpool.shape[0], float(rope_base), dt,
                                  _stream_handle(stream, k_new.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_kv_append_paged")


def attn_prefill_lse(q, k, v, scale=None, causal=True, out=None, lse=None, stream=None):
    """Prefill that also returns the row log-sum-exp lse [B,Hq,T] float32 (natural log)."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != T or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, Hkv, T, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = _empty((B, Hq, T, d), torch.float32, q.device, stream)
    if lse is None:
        lse = _empty((B, Hq, T), torch.float32, q.device, stream)
    if out.shape != q.shape or out.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, T) \
            or lse.dtype != torch.float32:
        raise ValueError("out must be float32 like q and lse float32 [B, Hq, T]")
    rc = lib.attn_prefill_lse(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                              _dev_ptr(lse, "lse"), B, Hq, Hkv, T, d, float(scale), int(bool(causal)),
                              _dtype_code(q), _stream_handle(stream, q.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_prefill_lse")
    return out, lse


def attn_backward_workspace_bytes(B, Hq, Hkv, T, d, dtype=GQA_BF16) -> int:
    return int(lib.attn_backward_workspace_bytes(B, Hq, Hkv, T, d, int(dtype)))


def attn_backward(q, k, v, out, dout, lse, scale=None, causal=True, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Gradients (dq, dk, dv) float32 of <dout, attention(q, k, v)> from the forward's
    out and lse (attn_prefill_lse); q, k, v float32 or bfloat16."""
    B, Hq, T, d = q.shape
    Hkv = k.shape[1]
    if k.dim() != 4 or k.shape[0] != B or k.shape[2] != T or k.shape[3] != d or v.shape != k.shape:
        raise ValueError("k, v must be [B, Hkv, T, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype")
    for t, n in ((out, "out"), (dout, "dout")):
        if t.shape != q.shape or t.dtype != torch.float32:
            raise ValueError("%s must be float32 of shape %s" % (n, tuple(q.shape)))
    if tuple(lse.shape) != (B, Hq, T) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Hq, T]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = _empty((B, Hq, T, d), torch.float32, q.device, stream) if dq is None else dq
    dk = _empty((B, Hkv, T, d), torch.float32, q.device, stream) if dk is None else dk
    dv = _empty((B, Hkv, T, d), torch.float32, q.device, stream) if dv is None else dv
    for t, n, shape in ((dq, "dq", (B, Hq, T, d)), (dk, "dk", (B, Hkv, T, d)), (dv, "dv", (B, Hkv, T, d))):
        if tuple(t.shape) != shape or t.dtype != torch.float32:
            raise ValueError("%s must be float32 of shape %s; got %s %s" % (n, shape, t.dtype, tuple(t.shape)))
    need = attn_backward_workspace_bytes(B, Hq, Hkv, T, d, _dtype_code(q))
    if workspace is None and need > 0:
        workspace = _empty(need, torch.uint8, q.device, stream)
    ws_ptr = _dev_ptr(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.attn_backward(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dev_ptr(out, "out"),
                           _dev_ptr(dout, "dout"), _dev_ptr(lse, "lse"), _dev_ptr(dq, "dq"), _dev_ptr(dk, "dk"),
                           _dev_ptr(dv, "dv"), B, Hq, Hkv, T, d, float(scale), int(bool(causal)), _dtype_code(q),
                           ws_ptr, ws_bytes, _stream_handle(stream, q.device))
    if rc != GQA_OK:
        raise GQAError(rc, "attn_backward")
    return dq, dk, dv
