"""C-ABI checks that need no GPU: the library loads, exports every function
include/gqa_attn.h declares, and rejects bad arguments on the host before any
launch (validation never touches the device, so these calls are safe without one).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")

gqa = pytest.importorskip("grouped_query_attention_amd")
lib = gqa.lib

EINVAL, EUNSUP, EWS, OK = gqa.GQA_EINVAL, gqa.GQA_EUNSUPPORTED, gqa.GQA_EWORKSPACE, gqa.GQA_OK
F32, BF16 = gqa.GQA_F32, gqa.GQA_BF16
A16 = 0x10000  # a 16-byte-aligned non-null fake pointer; never dereferenced (validation fails first
               # or the call has nothing to do)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported():
    names = header_functions()
    assert names, "no functions parsed from the header"
    assert sorted(gqa.EXPORTED) == names
    for n in names:
        assert hasattr(lib, n), n


def test_strerror():
    for code in (OK, EINVAL, EUNSUP, EWS, gqa.GQA_EHIP, 12345):
        s = gqa.attn_strerror(code)
        assert isinstance(s, str) and s


def prefill(q=A16, k=A16, v=A16, out=A16, B=1, Hq=2, Hkv=1, T=4, d=8, scale=0.5, causal=1, dtype=BF16,
            algo=0):
    return lib.attn_prefill_ex(q, k, v, out, B, Hq, Hkv, T, d, ctypes.c_float(scale), causal, dtype, algo,
                               None)


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=3, Hkv=2), EINVAL),            # Hq not a multiple of Hkv
    (dict(Hkv=0), EINVAL),
    (dict(Hq=0), EINVAL),
    (dict(B=-1), EINVAL),
    (dict(T=-1), EINVAL),
    (dict(d=0), EINVAL),
    (dict(d=257), EUNSUP),                  # no kernel beyond 256
    (dict(scale=float("inf")), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(causal=2), EINVAL),
    (dict(dtype=7), EINVAL),
    (dict(algo=9), EINVAL),
    (dict(q=None), EINVAL),                 # null pointer for a non-empty tensor
    (dict(out=A16 + 4), EINVAL),            # misaligned
    (dict(d=8, algo=2, dtype=F32), EUNSUP),  # fp32 matrix-core kernel: d a multiple of 16
    (dict(d=40, algo=2, dtype=F32), EUNSUP),
    (dict(d=160, algo=2, dtype=F32), EUNSUP),  # and at most 128
    (dict(d=8, algo=2), EUNSUP),            # d not a multiple of 16
])
def test_prefill_rejects(kw, code):
    assert prefill(**kw) == code


def test_prefill_empty_is_noop():
    # nothing to compute: returns OK without touching the (null) pointers
    assert prefill(q=None, k=None, v=None, out=None, B=0) == OK
    assert prefill(q=None, k=None, v=None, out=None, T=0) == OK


def decode(q=A16, kc=A16, vc=A16, out=A16, n=1, L=16, sp=15, Hq=4, Hkv=1, d=64, B=1, dtype=BF16, ws=A16,
           ws_bytes=1 << 30):
    return lib.attn_decode_cached(q, kc, vc, out, n, L, sp, Hq, Hkv, d, B, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(sp=16), EINVAL),         # startPos + newTokens > totalLen
    (dict(n=2, sp=15), EINVAL),
    (dict(sp=-1), EINVAL),
    (dict(n=-1), EINVAL),
    (dict(L=-1), EINVAL),
    (dict(Hq=6, Hkv=4), EINVAL),
    (dict(Hkv=0), EINVAL),
    (dict(d=0), EINVAL),
    (dict(d=300), EUNSUP),
    (dict(dtype=3), EINVAL),
    (dict(kc=None), EINVAL),
    (dict(vc=A16 + 2), EINVAL),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def test_decode_empty_is_noop():
    assert decode(q=None, kc=None, vc=None, out=None, n=0, sp=16) == OK
    assert decode(q=None, kc=None, vc=None, out=None, B=0) == OK


def test_decode_workspace_checked_before_launch():
    B, n, L, Hq, Hkv, d = 64, 4, 32768, 32, 8, 128
    need = gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, BF16)
    if need == 0:
        pytest.skip("this shape needs no workspace")
    args = dict(n=n, L=L, sp=L - n, Hq=Hq, Hkv=Hkv, d=d, B=B)
    assert decode(ws=None, ws_bytes=need, **args) == EWS
    assert decode(ws=A16, ws_bytes=need - 1, **args) == EWS
    assert decode(ws=A16 + 8, ws_bytes=need, **args) == EINVAL


def test_decode_plan_host_logic():
    """The split plan is a pure function of the shape: deterministic, at least one
    chunk, and the workspace covers one (max, sum, numerator) partial per chunk,
    query row and head dim when the history is split."""
    for (B, n, L, Hq, Hkv, d) in [(64, 1, 32768, 32, 8, 128), (64, 4, 32768, 32, 8, 128),
                                  (1, 1, 17, 4, 1, 64), (2, 3, 1000, 8, 2, 128), (1, 1, 1, 1, 1, 16)]:
        s1 = gqa.attn_decode_num_splits(B, n, L, Hq, Hkv, d, BF16)
        s2 = gqa.attn_decode_num_splits(B, n, L, Hq, Hkv, d, BF16)
        w = gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, BF16)
        assert s1 == s2 >= 1
        assert s1 <= L
        if s1 > 1:
            assert w >= s1 * B * n * Hq * (d + 2) * 4
        assert w == gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, BF16)
    # invalid shapes plan nothing
    assert gqa.attn_decode_num_splits(1, 2, 1, 4, 1, 64, BF16) == 0
    assert gqa.attn_decode_workspace_bytes(1, 1, 8, 3, 2, 64, BF16) == 0


def test_decode_plan_fills_the_simds():
    """The split plan aims at two waves per SIMD (1024 SIMDs) and, where the history is
    long enough to allow it, picks a chunk count whose waves fill the SIMDs to >= 90%
    (a partial last round of equal waves leaves SIMDs idle).  Chunks are whole 32-key
    tiles, so not every history admits such a count (1 x 100000 keys splits into 1563 or
    3125 chunks, both 76%); the shapes below all do."""
    simds = 1024
    for (B, n, L, Hq, Hkv, d) in [(64, 1, 32768, 32, 8, 128), (64, 4, 32768, 32, 8, 128), (48, 1, 32768, 32, 8, 128),
                                  (5, 1, 65536, 32, 8, 128), (1, 1, 98304, 8, 1, 64), (32, 2, 8192, 16, 4, 128)]:
        splits = gqa.attn_decode_num_splits(B, n, L, Hq, Hkv, d, BF16)
        units = B * Hkv * -(-((Hq // Hkv) * n) // 16)
        waves = units * splits
        assert waves >= simds, (B, n, L, splits)
        assert waves / (-(-waves // simds) * simds) >= 0.9, (B, n, L, splits, waves)
    # the contiguous 64-sequence, 32768-key cache: 8 KV heads x 64 sequences x 4 chunks = 2048 waves
    assert gqa.attn_decode_num_splits(64, 1, 32768, 32, 8, 128, BF16) == 4


A4 = 0x10004  # 4-byte aligned, not 16-byte aligned


def paged(q=A16, kp=A16, vp=A16, table=A16, lens=A16, out=A16, B=2, n=1, Hq=4, Hkv=1, d=64, bs=16,
          max_blocks=8, num_blocks=16, dtype=BF16, ws=A16, ws_bytes=1 << 30):
    return lib.attn_decode_paged(q, kp, vp, table, lens, out, B, n, Hq, Hkv, d, bs, max_blocks,
                                 num_blocks, dtype, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), EINVAL),
    (dict(B=-1), EINVAL),
    (dict(Hq=6, Hkv=4), EINVAL),
    (dict(Hkv=0), EINVAL),
    (dict(bs=0), EINVAL),
    (dict(bs=-16), EINVAL),
    (dict(max_blocks=0), EINVAL),
    (dict(num_blocks=0), EINVAL),
    (dict(bs=1 << 20, max_blocks=1 << 11), EINVAL),  # history longer than 2^30
    (dict(bs=24), EUNSUP),                           # block size not a multiple of 16
    (dict(dtype=F32), EUNSUP),                       # bf16 pools only
    (dict(d=72), EUNSUP),
    (dict(d=144), EUNSUP),
    (dict(dtype=5), EINVAL),
    (dict(table=None), EINVAL),
    (dict(lens=A16 + 2), EINVAL),
    (dict(kp=A4), EINVAL),
    (dict(out=None), EINVAL),
])
def test_paged_rejects(kw, code):
    assert paged(**kw) == code


def test_paged_table_and_lengths_need_only_4_byte_alignment():
    # validation passes with 4-byte aligned metadata; an empty call then does nothing
    assert paged(table=A4, lens=A4, B=0) == OK
    assert paged(q=None, kp=None, vp=None, table=None, lens=None, out=None, n=0) == OK
    assert paged(q=None, kp=None, vp=None, table=None, lens=None, out=None, B=0, bs=0,
                 max_blocks=0, num_blocks=0) == OK


def test_paged_workspace_checked_before_launch():
    B, n, Hq, Hkv, d, bs, mb = 64, 4, 32, 8, 128, 16, 2048
    need = gqa.attn_decode_paged_workspace_bytes(B, n, Hq, Hkv, d, bs, mb, BF16)
    assert need == gqa.attn_decode_workspace_bytes(B, n, bs * mb, Hq, Hkv, d, BF16) > 0
    args = dict(B=B, n=n, Hq=Hq, Hkv=Hkv, d=d, bs=bs, max_blocks=mb, num_blocks=B * mb)
    assert paged(ws=None, ws_bytes=need, **args) == EWS
    assert paged(ws=A16, ws_bytes=need - 1, **args) == EWS
    assert paged(ws=A16 + 8, ws_bytes=need, **args) == EINVAL
    # rejected shapes need nothing
    assert gqa.attn_decode_paged_workspace_bytes(B, n, Hq, Hkv, d, 24, mb, BF16) == 0
    assert gqa.attn_decode_paged_workspace_bytes(B, n, Hq, Hkv, d, bs, mb, F32) == 0


def test_window_entry_points_reject_bad_windows():
    f = ctypes.c_float(0.5)
    for w in (0, -1):
        assert lib.attn_prefill_window(A16, A16, A16, A16, 1, 2, 1, 8, 64, f, w, BF16, None) == EINVAL
        assert lib.attn_decode_window(A16, A16, A16, A16, 1, 16, 15, 4, 1, 64, 1, w, BF16, A16, 1 << 30,
                                      None) == EINVAL
        assert lib.attn_decode_paged_window(A16, A16, A16, A16, A16, A16, 2, 1, 4, 1, 64, 16, 8, 16, w,
                                            BF16, A16, 1 << 30, None) == EINVAL
        assert gqa.attn_decode_window_workspace_bytes(64, 1, 32768, 32, 8, 128, w) == 0
        assert gqa.attn_decode_paged_window_workspace_bytes(64, 1, 32, 8, 128, 16, 2048, w) == 0
    # the other checks still apply
    assert lib.attn_prefill_window(A16, A16, A16, A16, 1, 3, 2, 8, 64, f, 4, BF16, None) == EINVAL
    assert lib.attn_prefill_window(None, None, None, None, 0, 2, 1, 8, 64, f, 4, BF16, None) == OK


def test_window_workspace_follows_the_window():
    """The split plan of a window decode covers the window's keys, not the history."""
    B, n, L, Hq, Hkv, d = 64, 1, 32768, 32, 8, 128
    full = gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d)
    for W in (32, 1000, 4096):
        w = gqa.attn_decode_window_workspace_bytes(B, n, L, Hq, Hkv, d, W)
        assert 0 < w <= full
        p = gqa.attn_decode_paged_window_workspace_bytes(B, n, Hq, Hkv, d, 16, L // 16, W)
        assert p == w
    # a window wider than the history plans the history
    assert gqa.attn_decode_window_workspace_bytes(B, n, L, Hq, Hkv, d, 10 * L) == full


def kv_append(kn=A16, vn=A16, kc=A16, vc=A16, ff=None, B=1, n=2, Hkv=2, d=16, L=8, sp=6, base=10000.0,
              dtype=BF16):
    return lib.attn_kv_append(kn, vn, kc, vc, ff, B, n, Hkv, d, L, sp, ctypes.c_float(base), dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(sp=7), EINVAL),                   # start_pos + newTokens > totalLen
    (dict(sp=-1), EINVAL),
    (dict(n=-1), EINVAL),
    (dict(B=-1), EINVAL),
    (dict(Hkv=0), EINVAL),
    (dict(d=12), EUNSUP),                   # not a multiple of 8
    (dict(d=264), EUNSUP),
    (dict(base=-1.0), EINVAL),
    (dict(base=float("inf")), EINVAL),
    (dict(base=float("nan")), EINVAL),
    (dict(dtype=5), EINVAL),
    (dict(kc=None), EINVAL),
    (dict(vn=A16 + 4), EINVAL),             # misaligned
    (dict(ff=A16 + 2), EINVAL),             # freq factors not 4-byte aligned
    (dict(B=0), OK),                        # nothing to do
    (dict(n=0), OK),
])
def test_kv_append_rejects(kw, code):
    assert kv_append(**kw) == code


def test_kv_append_paged_rejects():
    def call(bs=16, mb=4, nb=8, table=A16, lens=A16, n=1, d=16):
        return lib.attn_kv_append_paged(A16, A16, A16, A16, table, lens, None, 2, n, 2, d, bs, mb, nb,
                                        ctypes.c_float(10000.0), BF16, None)
    assert call(bs=0) == EINVAL
    assert call(mb=0) == EINVAL
    assert call(nb=-1) == EINVAL
    assert call(table=None) == EINVAL
    assert call(lens=A16 + 2) == EINVAL
    assert call(d=20) == EUNSUP
    assert call(n=0) == OK
