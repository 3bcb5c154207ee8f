"""Parity at the benchmark's full sizes, in the launch configuration the benchmark times
(attn_prefill / attn_decode_cached with the default kernel choice), checked on sampled
outputs that the float64 oracle computes one by one.

Prefill: for sampled (batch, head) pairs, rows at tile edges, the middle and the end
of the sequence, plus random rows.  Decode: for sampled (sequence, K/V head) units,
every new token of every query head of the group, with the unit's cache regenerated
on the CPU from its seed.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1.5e-2}


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


@pytest.mark.parametrize("cfg", [si.GQA_T4096, si.BITNET3B_T2048], ids=lambda c: c.name)
def test_full_size_prefill_sampled_rows(gqa, cfg):
    q, k, v = si.prefill_config_inputs(cfg)
    print("prefill", cfg.name, flush=True)
    out = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), scale=cfg.scale, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(cfg.seed)
    G = cfg.Hq // cfg.Hkv
    T = cfg.T
    pairs = [(0, 0), (cfg.B - 1, cfg.Hq - 1), (int(rng.integers(cfg.B)), int(rng.integers(cfg.Hq)))]
    worst = 0.0
    for b, h in pairs:
        g = h // G
        rows = sorted(set([0, 1, 31, 32, 63, 64, 127, 128, 255, T // 2, T - 2, T - 1]
                          + rng.integers(0, T, 8).tolist()))
        kb = oracle.to_f64(k[b:b + 1, g:g + 1])
        vb = oracle.to_f64(v[b:b + 1, g:g + 1])
        got = out[b, h].cpu().double().numpy()
        for i in rows:
            want = oracle.attention(q[b:b + 1, h:h + 1, i:i + 1], kb[:, :, :i + 1], vb[:, :, :i + 1],
                                    cfg.scale, True, i)
            worst = max(worst, float(np.abs(got[i] - want[0, 0, 0]).max()))
    print("%s sampled max-abs error %.3g" % (cfg.name, worst))
    assert worst <= TOL[cfg.dtype], worst


@pytest.fixture(scope="module")
def decode_data():
    cfg = si.DECODE_L32768_N1
    print("generating the decode cache (2 x %.1f GiB)" % (cfg.kv_bytes() / 2 / 2**30), flush=True)
    _, kc, vc = si.decode_inputs(cfg.B, 1, cfg.Hq, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype, cfg.seed,
                                 device="cuda")
    return kc, vc


@pytest.mark.parametrize("cfg", [si.DECODE_L32768_N1, si.DECODE_L32768_N4], ids=lambda c: c.name)
def test_full_size_decode_sampled_units(gqa, decode_data, cfg):
    kc, vc = decode_data  # the cache does not depend on newTokens
    q = si.decode_query(cfg.B, cfg.n, cfg.Hq, cfg.d, cfg.dtype, cfg.seed)
    print("decode", cfg.name, flush=True)
    out = gqa.attn_decode_cached(q.cuda(), kc, vc, cfg.start_pos)
    torch.cuda.synchronize()
    G = cfg.Hq // cfg.Hkv
    worst = 0.0
    for b, g in [(0, 0), (37, 5), (cfg.B - 1, cfg.Hkv - 1)]:
        kb = si.decode_cache_chunk(cfg.seed, 0, b, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype)[g]
        vb = si.decode_cache_chunk(cfg.seed, 1, b, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype)[g]
        # the cache on the device is exactly the regenerated one
        assert torch.equal(kc[b, g, -3:].cpu(), kb[-3:]) and torch.equal(vc[b, g, :3].cpu(), vb[:3])
        heads = slice(g * G, (g + 1) * G)
        want = oracle.decode_cached(q[b:b + 1, :, heads], kb[None, None], vb[None, None], cfg.start_pos)
        got = out[b:b + 1, :, heads].cpu().double().numpy()
        worst = max(worst, float(np.abs(got - want).max()))
    print("%s sampled max-abs error %.3g" % (cfg.name, worst))
    assert worst <= TOL[cfg.dtype], worst


@pytest.mark.parametrize("cfg", [si.DECODE_L32768_N1, si.DECODE_L32768_N4], ids=lambda c: c.name)
def test_full_size_paged_decode(gqa, decode_data, cfg):
    """The same cache scattered into 16-position blocks in a random order: attn_decode_paged
    must give exactly attn_decode_cached's result (same kernels and split plan), and match
    the oracle on a sampled unit."""
    kc, vc = decode_data
    bs = 16
    print("paged pools for", cfg.name, flush=True)
    kp, vp, table, lens = si.paged_from_contiguous(kc, vc, bs, cfg.seed)
    q = si.decode_query(cfg.B, cfg.n, cfg.Hq, cfg.d, cfg.dtype, cfg.seed)
    a = gqa.attn_decode_cached(q.cuda(), kc, vc, cfg.start_pos)
    p = gqa.attn_decode_paged(q.cuda(), kp, vp, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, p)
    G = cfg.Hq // cfg.Hkv
    b, g = 21, 3
    kb = si.decode_cache_chunk(cfg.seed, 0, b, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype)[g]
    vb = si.decode_cache_chunk(cfg.seed, 1, b, cfg.Hkv, cfg.total_len, cfg.d, cfg.dtype)[g]
    heads = slice(g * G, (g + 1) * G)
    want = oracle.decode_cached(q[b:b + 1, :, heads], kb[None, None], vb[None, None], cfg.start_pos)
    err = float(np.abs(p[b:b + 1, :, heads].cpu().double().numpy() - want).max())
    print("%s paged sampled max-abs error %.3g" % (cfg.name, err))
    assert err <= TOL[cfg.dtype], err
    # the same blocks token-major (attn_decode_blocks): again exactly the contiguous result
    kt = kp.permute(0, 2, 1, 3).contiguous()
    del kp
    vt = vp.permute(0, 2, 1, 3).contiguous()
    del vp
    print("%s token-major blocks" % cfg.name, flush=True)
    t = gqa.attn_decode_blocks(q.cuda(), kt, vt, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, t)
    del kt, vt
