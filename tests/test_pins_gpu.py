"""The oracle's pins, applied to the GPU path through the C ABI.

Each pin below is also checked on the float64 oracle (tests/test_oracle.py); here every
kernel the library dispatches to (bf16 matrix cores with one or two heads per
workgroup, fp32 matrix cores, the vector kernel, split-KV decode and paged decode)
must satisfy it too:

* large logits: q scaled by 8 and by 64 (exact in bf16 and fp32), so the rows are
  peaky, the running max moves block after block and the lazy rescale runs; the
  result must still meet the oracle at the parity gates (Riftco "Verification":
  large logits);
* shift invariance: a key component shared by every key adds a per-row constant to
  the scores, which softmax removes;
* scale 0: uniform weights, so a causal row is the mean of the value rows up to its
  own position and a non-causal row the mean of all of them (closed form, float64
  cumulative means);
* a negative scale (an exact sign flip of q in the bf16 kernel);
* a single position: the output is the first value row, bit for bit;
* backward causality: perturbing keys after position t leaves dq of rows <= t bitwise
  unchanged, perturbing queries and upstream gradients before t leaves dk and dv of
  keys >= t bitwise unchanged (Riftco "Verification": no gradient influence from
  future positions);
* non-finite values in the future: the documented isolation of the tiled kernels
  (a NaN key never reaches an earlier row; a NaN value row reaches only rows of its
  own 32-position block, through 0 * NaN in that block's P V product) -- see the
  oracle's exclusion of masked keys, which isolates every earlier row.

Parity gates (the benchmark spec): max-abs 1e-4 for fp32 inputs, 1.5e-2 for bf16 inputs.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from oracle import backward as bw

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1.5e-2}
GENERIC, MFMA, AUTO, SPLIT = 1, 2, 0, 3
SEED = si.SEED_BASE + 700


def threads():
    return max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


def maxerr(got, want):
    return float(np.abs(got.detach().cpu().double().numpy() - want).max())


def prefill(gqa, q, k, v, scale, causal=True, algo=AUTO):
    out = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, algo=algo)
    torch.cuda.synchronize()
    return out


# (dtype, d, Hq, Hkv, algo): each row reaches a different kernel or instantiation
PREFILL_KERNELS = [
    ("bf16", 128, 4, 2, MFMA),    # matrix cores, two heads of a group per workgroup
    ("bf16", 80, 2, 2, MFMA),     # matrix cores, one head, padded P V head dims
    ("bf16", 64, 3, 1, MFMA),     # matrix cores, odd group: one head per workgroup
    ("bf16", 128, 2, 1, GENERIC),  # vector kernel
    ("bf16", 128, 4, 2, SPLIT),   # split-key matrix-core kernel
    ("bf16", 80, 2, 1, SPLIT),    # split-key, padded P V head dims
    ("f32", 64, 2, 2, MFMA),      # fp32 matrix cores
    ("f32", 128, 4, 2, MFMA),     # fp32 matrix cores, two heads per workgroup
    ("f32", 48, 2, 1, MFMA),      # fp32 matrix cores, padded head dims
    ("f32", 40, 2, 1, GENERIC),   # vector kernel
    ("f32", 64, 2, 2, SPLIT),     # fp32 split-key matrix-core kernel
    ("f32", 48, 2, 1, SPLIT),     # fp32 split-key, padded head dims
    ("f32", 128, 4, 2, SPLIT),    # fp32 split-key at the largest head dim
]


def kid(c):
    return "%s_d%d_Hq%d_Hkv%d_%s" % (c[0], c[1], c[2], c[3], {1: "generic", 2: "mfma", 0: "auto", 3: "split"}[c[4]])


@pytest.mark.parametrize("factor", [8, 64])
@pytest.mark.parametrize("kern", PREFILL_KERNELS, ids=kid)
def test_large_logits_prefill(gqa, kern, factor):
    dtype, d, Hq, Hkv, algo = kern
    T = 600  # several 128-key stages: interior (pipelined) and diagonal stages both run
    q, k, v = si.prefill_inputs(1, Hq, Hkv, T, d, dtype, SEED + d)
    q = q * factor  # a power of two: exact in bf16 and fp32
    scale = 1 / math.sqrt(d)
    want = oracle.prefill(q, k, v, scale, True, nthreads=threads())
    err = maxerr(prefill(gqa, q, k, v, scale, True, algo), want)
    print("q x %d %s max-abs %.3g" % (factor, kid(kern), err))
    assert err <= large_logit_tol(dtype, factor), err


def large_logit_tol(dtype, factor):
    """The parity gate for q scaled by `factor`.  bf16: the gate itself (the p rounding
    to bf16 dominates and does not grow with the scores).  fp32: the gate holds at q x 8;
    beyond that the float32 rounding of each score, which any fp32 evaluation carries,
    grows with the score's size (about sqrt(d) * 2^-24 * |s|, |s| here up to ~300), and
    the output error with it, so the bar is the gate scaled by factor / 8."""
    if dtype == "bf16":
        return TOL["bf16"]
    return TOL["f32"] * max(1.0, factor / 8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("factor", [8, 64])
@pytest.mark.parametrize("n", [1, 4])
def test_large_logits_decode(gqa, dtype, factor, n):
    B, Hq, Hkv, L, d = 2, 8, 2, 1000, 128
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dtype, SEED + n)
    q = q * factor
    want = oracle.decode_cached(q, kc, vc, L - n, nthreads=threads())
    got = gqa.attn_decode_cached(q.cuda(), kc.cuda(), vc.cuda(), L - n)
    torch.cuda.synchronize()
    err = maxerr(got, want)
    print("decode n=%d q x %d %s max-abs %.3g" % (n, factor, dtype, err))
    assert err <= large_logit_tol(dtype, factor), err


@pytest.mark.parametrize("factor", [8, 64])
@pytest.mark.parametrize("n", [1, 4])
def test_large_logits_paged_decode(gqa, factor, n):
    lens = [n, 300, 1500]
    q, kp, vp, tab, sl = si.paged_decode_inputs(3, n, 8, 2, 128, 16, lens, 100, "bf16", SEED + 10 * n,
                                                spare_blocks=2)
    q = q * factor
    want = oracle.decode_paged(q, kp, vp, tab, lens, 16)
    got = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), tab.cuda(), sl.cuda())
    torch.cuda.synchronize()
    err = maxerr(got, want)
    print("paged n=%d q x %d max-abs %.3g" % (n, factor, err))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("kern", PREFILL_KERNELS, ids=kid)
def test_shift_invariance_prefill(gqa, kern):
    """Key component d-1 is C for every key (0 in the reference): each score of row i
    gains scale * q[i, d-1] * C, a per-row constant (tens of units at C = 64)."""
    dtype, d, Hq, Hkv, algo = kern
    T = 300
    q, k, v = si.prefill_inputs(1, Hq, Hkv, T, d, dtype, SEED + 3 * d)
    k0 = k.clone()
    k0[..., -1] = 0
    ks = k.clone()
    ks[..., -1] = 64.0
    scale = 1 / math.sqrt(d)
    want = oracle.prefill(q, k0, v, scale, True, nthreads=threads())
    got = prefill(gqa, q, ks, v, scale, True, algo)
    err = maxerr(got, want)
    print("shift %s max-abs %.3g" % (kid(kern), err))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_shift_invariance_decode(gqa, dtype):
    B, n, Hq, Hkv, L, d = 2, 4, 8, 2, 700, 128
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dtype, SEED + 21)
    k0 = kc.clone()
    k0[..., -1] = 0
    ks = kc.clone()
    ks[..., -1] = 64.0
    want = oracle.decode_cached(q, k0, vc, L - n, nthreads=threads())
    got = gqa.attn_decode_cached(q.cuda(), ks.cuda(), vc.cuda(), L - n)
    torch.cuda.synchronize()
    assert maxerr(got, want) <= TOL[dtype]


def prefix_means(v, causal):
    """Closed form of scale 0: out[i] = mean(v[0..i]) (causal) or mean(v) (not)."""
    v = v.double().numpy()
    if causal:
        return np.cumsum(v, axis=2) / np.arange(1, v.shape[2] + 1)[:, None]
    return np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kern", PREFILL_KERNELS, ids=kid)
def test_scale_zero_is_prefix_mean(gqa, kern, causal):
    dtype, d, Hq, Hkv, algo = kern
    T = 333
    q, k, v = si.prefill_inputs(1, Hq, Hkv, T, d, dtype, SEED + 5 * d)
    got = prefill(gqa, q, k, v, 0.0, causal, algo)
    G = Hq // Hkv
    want = prefix_means(v, causal).repeat(G, axis=1)  # head h reads K/V head h // G
    err = maxerr(got, want)
    print("scale 0 %s causal=%s max-abs %.3g" % (kid(kern), causal, err))
    # every weight is exactly 1: only the fp32 accumulation of at most T values rounds
    assert err <= 1e-5, err


@pytest.mark.parametrize("kern", PREFILL_KERNELS, ids=kid)
def test_negative_scale(gqa, kern):
    dtype, d, Hq, Hkv, algo = kern
    T = 300
    q, k, v = si.prefill_inputs(1, Hq, Hkv, T, d, dtype, SEED + 7 * d)
    scale = -1.5 / math.sqrt(d)
    want = oracle.prefill(q, k, v, scale, True, nthreads=threads())
    err = maxerr(prefill(gqa, q, k, v, scale, True, algo), want)
    print("negative scale %s max-abs %.3g" % (kid(kern), err))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("kern", PREFILL_KERNELS, ids=kid)
def test_single_position_returns_first_value_exactly(gqa, kern):
    dtype, d, Hq, Hkv, algo = kern
    q, k, v = si.prefill_inputs(2, Hq, Hkv, 1, d, dtype, SEED + 9 * d)
    G = Hq // Hkv
    for causal in (True, False):
        got = prefill(gqa, q * 4, k, v, 1 / math.sqrt(d), causal, algo).cpu()
        want = v.float().repeat_interleave(G, 1)
        assert torch.equal(got, want), (kid(kern), causal)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_position_decode_and_paged(gqa, dtype):
    B, Hq, Hkv, d = 3, 8, 2, 128
    q, kc, vc = si.decode_inputs(B, 1, Hq, Hkv, 1, d, dtype, SEED + 31)
    got = gqa.attn_decode_cached(q.cuda(), kc.cuda(), vc.cuda(), 0).cpu()
    torch.cuda.synchronize()
    want = vc[:, :, 0].float().repeat_interleave(Hq // Hkv, 1)[:, None]  # [B, 1, Hq, d]
    assert torch.equal(got, want)
    if dtype == "bf16":
        q, kp, vp, tab, sl = si.paged_decode_inputs(B, 1, Hq, Hkv, d, 16, [1] * B, 2, "bf16", SEED + 32,
                                                    spare_blocks=1)
        got = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), tab.cuda(), sl.cuda()).cpu()
        torch.cuda.synchronize()
        for b in range(B):
            first = vp[int(tab[b, 0]), :, 0].float().repeat_interleave(Hq // Hkv, 0)  # [Hq, d]
            assert torch.equal(got[b, 0], first), b


# ------------------------------------------------------------------ backward causality
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 80), ("f32", 64)])
def test_backward_causality_bitwise(gqa, dtype, d):
    B, Hq, Hkv, T = 1, 4, 2, 200
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, SEED + 11 * d)
    g = torch.Generator().manual_seed(SEED + 12 * d)
    dout = torch.randn(B, Hq, T, d, generator=g, dtype=torch.float32)
    scale = 1 / math.sqrt(d)

    def grads(q_, k_, v_, do_):
        qd, kd, vd = q_.cuda(), k_.cuda(), v_.cuda()
        out, lse = gqa.attn_prefill_lse(qd, kd, vd, scale=scale, causal=True)
        r = gqa.attn_backward(qd, kd, vd, out, do_.cuda(), lse, scale=scale, causal=True)
        torch.cuda.synchronize()
        return [x.cpu() for x in r]

    dq, dk, dv = grads(q, k, v, dout)
    for t in (0, 31, 32, 100, 150):
        # keys and values after t: dq of rows <= t must not move
        k2, v2 = k.clone(), v.clone()
        k2[:, :, t + 1:] = -2 * k2[:, :, t + 1:]
        v2[:, :, t + 1:] = 3 * v2[:, :, t + 1:] + 1
        dq2, _, _ = grads(q, k2, v2, dout)
        assert torch.equal(dq2[:, :, :t + 1], dq[:, :, :t + 1]), ("dq", t)
        # queries and upstream gradients before t: dk, dv of keys >= t must not move
        q3, do3 = q.clone(), dout.clone()
        q3[:, :, :t] = 2 * q3[:, :, :t] - 1
        do3[:, :, :t] = -5 * do3[:, :, :t]
        _, dk3, dv3 = grads(q3, k, v, do3)
        assert torch.equal(dk3[:, :, t:], dk[:, :, t:]), ("dk", t)
        assert torch.equal(dv3[:, :, t:], dv[:, :, t:]), ("dv", t)
    # the unperturbed gradients still meet the oracle
    want = bw.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                       scale, True)
    rel = 1.5e-2 if dtype == "bf16" else 1e-4
    for got, ref in zip((dq, dk, dv), want):
        assert np.abs(got.double().numpy() - ref).max() <= rel * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------- non-finite isolation
@pytest.mark.parametrize("kern", PREFILL_KERNELS, ids=kid)
def test_nan_isolation_prefill(gqa, kern):
    """A NaN in a future key never reaches an earlier row (its score is replaced by the
    mask before the softmax).  A NaN in a future value row at position j never reaches
    rows before its 32-position block (32 * (j // 32)); rows inside that block may turn
    NaN through 0 * NaN in the block's P V product.  The oracle excludes masked keys
    and so isolates every earlier row."""
    dtype, d, Hq, Hkv, algo = kern
    T = 260
    q, k, v = si.prefill_inputs(1, Hq, Hkv, T, d, dtype, SEED + 13 * d)
    scale = 1 / math.sqrt(d)
    base = prefill(gqa, q, k, v, scale, True, algo).cpu()
    for j in (40, 127, 128, 200):
        k2 = k.clone()
        k2[:, :, j] = float("nan")
        got = prefill(gqa, q, k2, v, scale, True, algo).cpu()
        assert torch.equal(got[:, :, :j], base[:, :, :j]), ("key", j)
        assert torch.isnan(got[:, :, j:]).all(), ("key", j)
        v2 = v.clone()
        v2[:, :, j] = float("nan")
        got = prefill(gqa, q, k, v2, scale, True, algo).cpu()
        blk = 32 * (j // 32)
        assert torch.equal(got[:, :, :blk], base[:, :, :blk]), ("value", j)
        assert torch.isnan(got[:, :, j:]).all(), ("value", j)
    # the oracle: every earlier row is isolated
    k2 = k.clone()
    k2[:, :, 150] = float("nan")
    v2 = v.clone()
    v2[:, :, 150] = float("nan")
    o = oracle.prefill(q, k2, v2, scale, True, nthreads=threads())
    ob = oracle.prefill(q, k, v, scale, True, nthreads=threads())
    assert np.array_equal(o[:, :, :150], ob[:, :, :150]) and np.isnan(o[:, :, 150:]).all()


# --------------------------------------------------------------------- guard bands
@pytest.mark.parametrize("dtype,d,Hq,Hkv", [("f32", 48, 4, 2), ("f32", 128, 4, 2), ("f32", 40, 2, 1),
                                            ("bf16", 64, 3, 1)])
def test_prefill_output_guard_bands(gqa, dtype, d, Hq, Hkv):
    B, T = 2, 77
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, SEED + 15 * d)
    n, pad = B * Hq * T * d, 4096
    buf = torch.full((n + 2 * pad,), 7.25, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + n].view(B, Hq, T, d)
    gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 7.25) and torch.all(buf[pad + n:] == 7.25)
    assert maxerr(out, oracle.prefill(q, k, v, 1 / math.sqrt(d), True, nthreads=threads())) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n", [1, 4])
def test_decode_guard_bands(gqa, dtype, n):
    """out and the workspace are written only inside their extents: sentinels on both
    sides of each stay untouched."""
    B, Hq, Hkv, L, d = 3, 16, 4, 2500, 128
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dtype, SEED + 17 * n)
    no, pad = B * n * Hq * d, 4096
    obuf = torch.full((no + 2 * pad,), -3.5, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + no].view(B, n, Hq, d)
    need = gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, gqa.GQA_BF16 if dtype == "bf16" else gqa.GQA_F32)
    wpad = 4096
    wbuf = torch.full((need + 2 * wpad,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = wbuf[wpad:wpad + need] if need else None
    gqa.attn_decode_cached(q.cuda(), kc.cuda(), vc.cuda(), L - n, out=out, workspace=ws)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == -3.5) and torch.all(obuf[pad + no:] == -3.5)
    assert torch.all(wbuf[:wpad] == 0xA5) and torch.all(wbuf[wpad + need:] == 0xA5)
    assert maxerr(out, oracle.decode_cached(q, kc, vc, L - n, nthreads=threads())) <= TOL[dtype]


def test_paged_decode_guard_bands(gqa):
    n, lens = 4, [4, 700, 1300]
    q, kp, vp, tab, sl = si.paged_decode_inputs(3, n, 16, 4, 128, 32, lens, 60, "bf16", SEED + 19,
                                                spare_blocks=2)
    B, Hq, d = 3, 16, 128
    no, pad = B * n * Hq * d, 4096
    obuf = torch.full((no + 2 * pad,), -3.5, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + no].view(B, n, Hq, d)
    need = gqa.attn_decode_paged_workspace_bytes(B, n, Hq, 4, d, 32, 60)
    wbuf = torch.full((need + 2 * pad,), 0x5A, dtype=torch.uint8, device="cuda")
    gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), tab.cuda(), sl.cuda(), out=out,
                          workspace=wbuf[pad:pad + need])
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == -3.5) and torch.all(obuf[pad + no:] == -3.5)
    assert torch.all(wbuf[:pad] == 0x5A) and torch.all(wbuf[pad + need:] == 0x5A)
    assert maxerr(out, oracle.decode_paged(q, kp, vp, tab, lens, 32)) <= TOL["bf16"]


# ------------------------------------------------------------------- side streams
def test_calls_on_a_side_stream(gqa):
    """Every entry point on a caller's stream other than the current one, with the
    workspaces and outputs the binding allocates itself: results match the oracle."""
    s = torch.cuda.Stream()
    q, k, v = si.prefill_inputs(1, 4, 2, 300, 128, "bf16", SEED + 41)
    qd_, kc, vc = si.decode_inputs(2, 4, 8, 2, 3000, 128, "bf16", SEED + 42)
    g = torch.Generator().manual_seed(SEED + 43)
    dout = torch.randn(q.shape, generator=g, dtype=torch.float32)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # inputs made on the side stream's side of the fence
        dq_, dk_, dv_ = q.cuda(), k.cuda(), v.cuda()
        qd, kcd, vcd, dod = qd_.cuda(), kc.cuda(), vc.cuda(), dout.cuda()
    s.synchronize()
    outs = []
    for rep in range(3):  # repeated calls reuse freed blocks: any race would show
        o = gqa.attn_decode_cached(qd, kcd, vcd, 3000 - 4, stream=s)
        p = gqa.attn_prefill(dq_, dk_, dv_, stream=s)
        pl, lse = gqa.attn_prefill_lse(dq_, dk_, dv_, stream=s)
        gr = gqa.attn_backward(dq_, dk_, dv_, pl, dod, lse, stream=s)
        outs.append((o, p, gr))
    s.synchronize()
    want_d = oracle.decode_cached(qd_, kc, vc, 3000 - 4, nthreads=threads())
    want_p = oracle.prefill(q, k, v, 1 / math.sqrt(128), True, nthreads=threads())
    want_g = bw.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                         1 / math.sqrt(128), True)
    for o, p, gr in outs:
        assert maxerr(o, want_d) <= TOL["bf16"]
        assert maxerr(p, want_p) <= TOL["bf16"]
        for got, ref in zip(gr, want_g):
            assert maxerr(got, ref) <= 1.5e-2 * max(1.0, np.abs(ref).max())
