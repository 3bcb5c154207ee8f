"""Parity at the benchmark's full sizes, in the launch configuration the benchmark times
(attn_prefill / attn_decode_cached with the default kernel choice, preallocated out),
compared with the float64 oracle on every output element.

* GQA prefill (B=2, 16 query / 8 K/V heads, T=4096, d=128) and the BitNet-3B attention
  shape (B=8, 32 heads of d=80, T=2048): the whole output against the threaded C oracle.
* Cached decode (64 sequences, 32 query / 8 K/V heads, d=128, a 32768-position bf16
  cache), newTokens 1 and 4: every sequence, every K/V head and every query head, the
  oracle fed one sequence at a time from the device cache (checked to be the seeded
  one).
* Paged and token-major block decode over the same cache scattered into 16-position
  blocks: bitwise equal to the contiguous call, so the exhaustive check carries over.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1.5e-2}


def threads():
    return max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


@pytest.mark.parametrize("cfg", [si.GQA_T4096, si.BITNET3B_T2048], ids=lambda c: c.name)
def test_full_size_prefill_every_element(gqa, cfg):
    q, k, v = si.prefill_config_inputs(cfg)
    print("prefill", cfg.name, flush=True)
    out = torch.empty((cfg.B, cfg.Hq, cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), scale=cfg.scale, causal=True, out=out)
    got = out.cpu().double().numpy()
    del out
    print("oracle", cfg.name, flush=True)
    want = oracle.prefill(q, k, v, cfg.scale, True, nthreads=threads())
    diff = np.abs(got - want)
    err = float(diff.max())
    rms = float(np.sqrt((diff ** 2).mean()))
    print("%s every element: max-abs %.3g, rms %.3g" % (cfg.name, err, rms))
    assert err <= TOL[cfg.dtype], err


@pytest.fixture(scope="module")
def decode_data():
    cfg = si.DECODE_L32768_N1
    print("generating the decode cache (2 x %.1f GiB)" % (cfg.kv_bytes() / 2 / 2**30), flush=True)
    _, kc, vc = si.decode_inputs(cfg.B, 1, cfg.Hq, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype, cfg.seed,
                                 device="cuda")
    return kc, vc


def test_full_size_decode_every_sequence(gqa, decode_data):
    kc, vc = decode_data
    c1, c4 = si.DECODE_L32768_N1, si.DECODE_L32768_N4
    outs, qs = {}, {}
    for cfg in (c1, c4):
        qs[cfg.n] = si.decode_query(cfg.B, cfg.n, cfg.Hq, cfg.d, cfg.dtype, cfg.seed)
        out = torch.empty((cfg.B, cfg.n, cfg.Hq, cfg.d), dtype=torch.float32, device="cuda")
        ws = torch.empty(gqa.attn_decode_workspace_bytes(cfg.B, cfg.n, cfg.total_len, cfg.Hq, cfg.Hkv, cfg.d),
                         dtype=torch.uint8, device="cuda")
        print("decode", cfg.name, flush=True)
        gqa.attn_decode_cached(qs[cfg.n].cuda(), kc, vc, cfg.start_pos, out=out, workspace=ws)
        outs[cfg.n] = out.cpu().double().numpy()
    worst = {1: 0.0, 4: 0.0}
    for b in range(c1.B):
        if b % 16 == 0:
            print("oracle over sequences %d.." % b, flush=True)
        if b in (0, 37, c1.B - 1):  # the device cache is the seeded one
            kb = si.decode_cache_chunk(c1.seed, 0, b, c1.Hkv, c1.total_len, c1.d, c1.dtype)
            vb = si.decode_cache_chunk(c1.seed, 1, b, c1.Hkv, c1.total_len, c1.d, c1.dtype)
            assert torch.equal(kc[b].cpu(), kb) and torch.equal(vc[b].cpu(), vb), b
        k64 = kc[b].cpu().double().numpy()[None]
        v64 = vc[b].cpu().double().numpy()[None]
        for cfg in (c1, c4):
            want = oracle.decode_cached(qs[cfg.n][b:b + 1], k64, v64, cfg.start_pos, nthreads=threads())
            worst[cfg.n] = max(worst[cfg.n], float(np.abs(outs[cfg.n][b:b + 1] - want).max()))
    print("decode every unit: max-abs n=1 %.3g, n=4 %.3g" % (worst[1], worst[4]))
    assert worst[1] <= TOL[c1.dtype] and worst[4] <= TOL[c4.dtype], worst


@pytest.mark.parametrize("cfg", [si.DECODE_L32768_N1, si.DECODE_L32768_N4], ids=lambda c: c.name)
def test_full_size_paged_and_blocks_equal_contiguous(gqa, decode_data, cfg):
    """The same cache scattered into 16-position blocks in a random order: attn_decode_paged
    and attn_decode_blocks (token-major blocks) give exactly attn_decode_cached's result
    (same kernels and split plan), which the test above checks on every element."""
    kc, vc = decode_data
    bs = 16
    print("paged pools for", cfg.name, flush=True)
    kp, vp, table, lens = si.paged_from_contiguous(kc, vc, bs, cfg.seed)
    q = si.decode_query(cfg.B, cfg.n, cfg.Hq, cfg.d, cfg.dtype, cfg.seed).cuda()
    a = gqa.attn_decode_cached(q, kc, vc, cfg.start_pos)
    p = gqa.attn_decode_paged(q, kp, vp, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, p)
    kt = kp.permute(0, 2, 1, 3).contiguous()
    del kp
    vt = vp.permute(0, 2, 1, 3).contiguous()
    del vp
    print("%s token-major blocks" % cfg.name, flush=True)
    t = gqa.attn_decode_blocks(q, kt, vt, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, t)
    del kt, vt
