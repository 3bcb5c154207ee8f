"""Local (sliding-window) causal attention on the GPU against the float64 oracle.

attn_prefill_window, attn_decode_window and attn_decode_paged_window restrict query
position p to keys p-W+1 .. p (the multi-query primer's local attention, section 4.1,
uses W = 32).  Checked here: element-wise parity on the matrix-core and vector-ALU
kernels with windows below, at and across tile (64) and stage (128) sizes, ragged
lengths and G = 1..4; W = 1 returns each row's own value; W >= T equals plain causal
bitwise; cache rows and table entries below the window are never read (they hold NaN
or -1 here).
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


PREFILL = [
    # B, Hq, Hkv, T, d, W, dtype
    (1, 4, 2, 300, 128, 32, "bf16"),
    (2, 4, 4, 777, 64, 100, "bf16"),
    (1, 2, 1, 1000, 80, 256, "bf16"),
    (1, 4, 2, 513, 128, 129, "bf16"),
    (1, 4, 2, 700, 128, 64, "bf16"),
    (1, 4, 2, 700, 128, 128, "bf16"),
    (1, 3, 1, 600, 128, 200, "bf16"),
    (1, 4, 2, 130, 64, 17, "f32"),
    (1, 2, 1, 100, 24, 10, "bf16"),
    (2, 8, 2, 2048, 128, 1000, "bf16"),
    (1, 4, 2, 300, 128, 100, "f32"),   # fp32 matrix cores, two heads of a group per workgroup
    (1, 4, 2, 260, 112, 70, "f32"),    # fp32 matrix cores, padded head dims, head pairs
]


def pid(c):
    return "B%dHq%dHkv%dT%dd%dW%d-%s" % c


@pytest.mark.parametrize("case", PREFILL, ids=pid)
def test_window_prefill_matches_oracle(gqa, case):
    B, Hq, Hkv, T, d, W, dt = case
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dt, seed=3100 + T + W)
    scale = d ** -0.5
    print("window prefill", pid(case), flush=True)
    out = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), scale=scale, window=W)
    torch.cuda.synchronize()
    want = oracle.prefill(q, k, v, scale, True, window=W)
    err = float(np.abs(out.cpu().double().numpy() - want).max())
    print("max-abs error %.3g" % err)
    assert err <= TOL[dt], err


@pytest.mark.parametrize("d", [64, 128, 24])
def test_window_one_is_own_value(gqa, d):
    q, k, v = si.prefill_inputs(1, 4, 2, 200, d, "bf16", seed=3200 + d)
    out = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), scale=0.3, window=1)
    torch.cuda.synchronize()
    want = v.float().repeat_interleave(2, dim=1)
    assert torch.equal(out.cpu(), want)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 80), ("f32", 128), ("f32", 48)])
def test_wide_window_is_causal_bitwise(gqa, dtype, d):
    # a window reaching key 0 from every row takes the causal call's kernel (at this
    # small shape the split-key kernel, in either dtype)
    q, k, v = si.prefill_inputs(1, 4, 2, 333, d, dtype, seed=3300 + d)
    qc, kc, vc = q.cuda(), k.cuda(), v.cuda()
    a = gqa.attn_prefill(qc, kc, vc, scale=d ** -0.5)
    for W in (333, 334, 100000):
        b = gqa.attn_prefill(qc, kc, vc, scale=d ** -0.5, window=W)
        torch.cuda.synchronize()
        assert torch.equal(a, b), W


DECODE = [
    # B, n, Hq, Hkv, L, d, W, dtype
    (2, 1, 8, 2, 3000, 128, 32, "bf16"),
    (2, 4, 16, 4, 5000, 128, 1000, "bf16"),
    (1, 3, 4, 1, 700, 64, 700, "bf16"),
    (1, 2, 4, 4, 100, 80, 7, "bf16"),
    (3, 1, 32, 8, 4096, 128, 4096, "bf16"),
    (1, 5, 8, 2, 2000, 128, 1, "bf16"),
    (1, 2, 4, 2, 300, 64, 50, "f32"),
]


def did(c):
    return "B%dn%dHq%dHkv%dL%dd%dW%d-%s" % c


@pytest.mark.parametrize("case", DECODE, ids=did)
def test_window_decode_matches_oracle(gqa, case):
    B, n, Hq, Hkv, L, d, W, dt = case
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dt, seed=3400 + L + W)
    start = L - n
    want = oracle.decode_cached(q, kc, vc, start, window=W)
    # rows below the first window start (rounded down to 32) must never be read
    lo = max(0, (start - W + 1) // 32 * 32)
    kg, vg = kc.clone(), vc.clone()
    kg[:, :, :lo] = float("nan")
    vg[:, :, :lo] = float("nan")
    print("window decode", did(case), flush=True)
    out = gqa.attn_decode_cached(q.cuda(), kg.cuda(), vg.cuda(), start, window=W)
    torch.cuda.synchronize()
    err = float(np.abs(out.cpu().double().numpy() - want).max())
    print("max-abs error %.3g" % err)
    assert err <= TOL[dt], err


def test_window_decode_start_inside_cache(gqa):
    B, n, Hq, Hkv, L, d, W = 2, 3, 8, 2, 1200, 128, 300
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, "bf16", seed=3500)
    start = 800  # rows 803.. are never read
    kc[:, :, start + n:] = float("nan")
    vc[:, :, start + n:] = float("nan")
    want = oracle.decode_cached(q, kc[:, :, :start + n], vc[:, :, :start + n], start, window=W)
    out = gqa.attn_decode_cached(q.cuda(), kc.cuda(), vc.cuda(), start, window=W)
    torch.cuda.synchronize()
    assert float(np.abs(out.cpu().double().numpy() - want).max()) <= TOL["bf16"]


PAGED = [
    # B, n, Hq, Hkv, d, bs, lens, max_blocks, W
    (3, 2, 8, 2, 128, 16, [50, 700, 3000], 200, 100),
    (2, 1, 16, 4, 64, 32, [4000, 33], 130, 32),
    (2, 4, 8, 8, 128, 48, [1000, 500], 30, 400),
    (1, 1, 4, 1, 80, 256, [5000], 20, 2000),
]


@pytest.mark.parametrize("case", PAGED, ids=lambda c: "B%dn%dbs%dW%d-L%s" % (c[0], c[1], c[5], c[8],
                                                                         "_".join(map(str, c[6]))))
def test_window_paged_matches_oracle(gqa, case):
    B, n, Hq, Hkv, d, bs, lens, mb, W = case
    q, kp, vp, table, sl = si.paged_decode_inputs(B, n, Hq, Hkv, d, bs, lens, mb, "bf16",
                                                  seed=3600 + W, spare_blocks=2)
    want = oracle.decode_paged(q, kp, vp, table, lens, bs, window=W)
    # table entries of blocks wholly below the first window start (rounded down to 32)
    # are never read
    t2 = table.clone()
    for b, L in enumerate(lens):
        lo = max(0, (L - n - W + 1) // 32 * 32)
        t2[b, :lo // bs] = -1
    print("window paged", lens, W, flush=True)
    out = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), t2.cuda(), sl.cuda(), window=W)
    torch.cuda.synchronize()
    err = float(np.abs(out.cpu().double().numpy() - want).max())
    print("max-abs error %.3g" % err)
    assert err <= TOL["bf16"], err
