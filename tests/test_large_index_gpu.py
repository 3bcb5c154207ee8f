"""Tensors whose element offsets pass the 32-bit range.

* Prefill with q and out of more than 2^31 elements (B=36, 64 query / 8 K/V heads,
  T=8192, d=128, causal), bf16 and fp32 inputs, on the one-workgroup-per-q-tile kernels
  (the automatic choice at this size).
* Cached decode over a cache of 2^32 elements per tensor (64 sequences, 8 K/V heads,
  65536 positions, d=128, bf16), newTokens 1; then the same history scattered in
  16-position blocks over a pool of the same size, through the paged call.

The inputs are seeded N(0,1) draws made on the device (host memory would need tens of
GB).  Sampled output rows at the far end of the tensors, the very last one included,
are compared with the float64 oracle fed exactly those rows' inputs, copied back.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1.5e-2}
SEED = 20261204


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


def device_normal(shape, seed, dtype):
    """Seeded N(0,1) on the GPU, drawn in fp32 one leading index at a time and rounded to
    `dtype` (bf16 by round-to-nearest-even)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device="cuda")
    for i in range(shape[0]):
        out[i] = torch.randn(shape[1:], generator=g, device="cuda", dtype=torch.float32).to(dtype)
    return out


def oracle_row(q, k, v, b, h, i, G, scale):
    """Oracle output of query row i of head h in sequence b (keys 0..i of K/V head h // G)."""
    qr = q[b, h, i].cpu().reshape(1, 1, 1, -1)
    kr = k[b, h // G, :i + 1].cpu().unsqueeze(0).unsqueeze(0)
    vr = v[b, h // G, :i + 1].cpu().unsqueeze(0).unsqueeze(0)
    return oracle.attention(qr, kr, vr, scale, True, pos0=i)[0, 0, 0]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_past_2g_elements(gqa, dtype):
    B, Hq, Hkv, T, d = 36, 64, 8, 8192, 128
    assert B * Hq * T * d > 2 ** 31
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = device_normal((B, Hq, T, d), SEED, tdt)
    k = device_normal((B, Hkv, T, d), SEED + 1, tdt)
    v = device_normal((B, Hkv, T, d), SEED + 2, tdt)
    scale = d ** -0.5
    print("prefill %s B=%d Hq=%d Hkv=%d T=%d d=%d" % (dtype, B, Hq, Hkv, T, d), flush=True)
    out = gqa.attn_prefill(q, k, v, scale=scale, causal=True)
    torch.cuda.synchronize()
    G = Hq // Hkv
    rng = np.random.default_rng(SEED)
    picks = [(B - 1, Hq - 1, T - 1), (B - 1, Hq - 1, T - 2), (B - 1, Hq - 2, T - 1), (B - 1, 0, T - 1),
             (B - 1, Hq - 1, 0), (B - 2, Hq - 1, T - 1)]
    picks += [(int(rng.integers(B // 2, B)), int(rng.integers(0, Hq)), int(rng.integers(0, T))) for _ in range(6)]
    for b, h, i in picks:
        want = oracle_row(q, k, v, b, h, i, G, scale)
        err = float(np.abs(out[b, h, i].cpu().double().numpy() - want).max())
        assert err <= TOL[dtype], (b, h, i, err)
    del q, k, v, out
    torch.cuda.empty_cache()


def test_decode_past_2g_elements(gqa):
    B, Hq, Hkv, L, d, n = 64, 32, 8, 65536, 128, 1
    assert B * Hkv * L * d > 2 ** 31
    kc = device_normal((B, Hkv, L, d), SEED + 3, torch.bfloat16)
    vc = device_normal((B, Hkv, L, d), SEED + 4, torch.bfloat16)
    q = device_normal((B, n, Hq, d), SEED + 5, torch.bfloat16)
    print("decode B=%d Hq=%d Hkv=%d L=%d d=%d n=%d" % (B, Hq, Hkv, L, d, n), flush=True)
    out = gqa.attn_decode_cached(q, kc, vc, L - n)
    torch.cuda.synchronize()
    for b in (B - 1, B - 2, 0):
        want = oracle.decode_cached(q[b:b + 1].cpu(), kc[b:b + 1].cpu(), vc[b:b + 1].cpu(), L - n,
                                    nthreads=max(1, min(16, os.cpu_count() or 1)))
        err = float(np.abs(out[b:b + 1].cpu().double().numpy() - want).max())
        assert err <= TOL["bf16"], (b, err)
    # the same history in 16-position blocks of a pool of 2^32 elements per tensor, in
    # seeded random order: the paged call reads the same rows, so it is bitwise the same
    kp, vp, table, lens = si.paged_from_contiguous(kc, vc, 16, SEED + 6)
    del kc, vc
    torch.cuda.empty_cache()
    print("paged decode over a pool of %d blocks" % kp.shape[0], flush=True)
    paged = gqa.attn_decode_paged(q, kp, vp, table, lens)
    torch.cuda.synchronize()
    assert torch.equal(paged, out)
    del kp, vp, q, out, paged
    torch.cuda.empty_cache()
