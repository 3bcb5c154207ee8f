"""Row statistics (attn_prefill_lse) and the backward pass (attn_backward) on the GPU
against the float64 oracle (oracle/backward.py).

* lse from the forward kernels (bf16 matrix cores, split-key bf16 matrix cores for small
  shapes, fp32 matrix cores, and the vector kernel for head dims those do not take) against
  the oracle's row log-sum-exp; the output is bitwise that of attn_prefill.
* dq, dk, dv element by element against the oracle on ragged shapes (T not a multiple
  of the 32/64/128-row tiles), every head dim the matrix-core path takes (16..128 in
  steps of 16), group sizes 1, 2, 4, causal and not, and at the full GQA prefill workload on every
  head group.
  The GPU recomputes P from bf16 Q/K, rounds P, dS and dO to bf16 for the matrix cores
  and accumulates in fp32; the bar is the bf16-input tolerance 1.5e-2 applied to the
  gradient scaled by its own size: max|gpu - ref| <= 1.5e-2 * max(1, max|ref|).
* the vector-ALU backward (fp32 inputs, and bf16 head dims that are not a multiple of
  16) against the same oracle: 1e-4 scaled the same way for fp32 inputs.
* the oracle's invariants hold on the GPU result: key gradients of a K/V head sum to
  ~0 over the keys, value gradients sum to the upstream gradient.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from oracle import backward as bw

pytestmark = pytest.mark.gpu

SEED = si.SEED_BASE + 50


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


def inputs(B, Hq, Hkv, T, d, dtype, seed):
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    dout = torch.randn(B, Hq, T, d, generator=g, dtype=torch.float32)
    return q, k, v, dout


def close(got, want, rel=1.5e-2):
    got = got.double().cpu().numpy() if torch.is_tensor(got) else got
    err = np.abs(got - want).max()
    bound = rel * max(1.0, np.abs(want).max())
    assert err <= bound, (float(err), float(bound))
    return err


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("bf16", 64, False), ("bf16", 80, True),
                                            ("f32", 64, True), ("f32", 40, False)])
def test_lse_matches_oracle(gqa, dtype, d, causal):
    B, Hq, Hkv, T = 2, 4, 2, 197
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, SEED + d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, lse = gqa.attn_prefill_lse(qd, kd, vd, scale=d ** -0.5, causal=causal)
    ref_out = gqa.attn_prefill(qd, kd, vd, scale=d ** -0.5, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    want = bw.lse(q.double().numpy(), k.double().numpy(), d ** -0.5, causal)
    tol = 1.5e-2 if dtype == "bf16" else 1e-4
    assert np.abs(lse.cpu().double().numpy() - want).max() <= tol


def test_lse_worked_example(gqa):
    """The primer's example through the fp32 kernel: row 2 of q = (1,0) over keys
    (1,0), (0,1), (1,1), unscaled: lse = log(2e + 1)."""
    q = torch.zeros(1, 1, 3, 2)
    q[0, 0, 2] = torch.tensor([1.0, 0.0])
    k = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).reshape(1, 1, 3, 2)
    v = torch.tensor([[1.0, 0.0], [2.0, 0.0], [3.0, 0.0]]).reshape(1, 1, 3, 2)
    out, lse = gqa.attn_prefill_lse(q.cuda(), k.cuda(), v.cuda(), scale=1.0, causal=True)
    torch.cuda.synchronize()
    assert abs(lse[0, 0, 2].item() - math.log(2 * math.e + 1)) <= 1e-6
    assert abs(out[0, 0, 2, 0].item() - 2.0) <= 1e-6


CASES = [
    # B, Hq, Hkv, T, d, causal
    (2, 4, 2, 200, 128, True),
    (1, 4, 1, 333, 64, True),
    (2, 2, 2, 130, 80, True),
    (1, 8, 2, 257, 32, False),
    (2, 3, 3, 64, 128, False),
    (1, 2, 1, 45, 16, True),
    (1, 16, 8, 512, 128, True),
    (1, 2, 2, 1, 64, True),
    (1, 4, 2, 150, 48, True),
    (2, 2, 1, 97, 96, False),
    (1, 4, 2, 222, 112, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_T%d_d%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], "causal" if c[5] else "full"))
def test_backward_matches_oracle(gqa, case):
    B, Hq, Hkv, T, d, causal = case
    q, k, v, dout = inputs(B, Hq, Hkv, T, d, "bf16", SEED + 7 * T + d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = d ** -0.5
    out, lse = gqa.attn_prefill_lse(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = gqa.attn_backward(qd, kd, vd, out, dout.cuda(), lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    wq, wk, wv = bw.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                             scale, causal)
    close(dq, wq)
    close(dk, wk)
    close(dv, wv)
    # invariants of the exact gradients hold to the same bar
    G = Hq // Hkv
    dks = dk.double().cpu().numpy().sum(axis=2)
    assert np.abs(dks).max() <= 1.5e-2 * max(1.0, np.abs(wk).max()) * math.sqrt(T)
    dvs = dv.double().cpu().numpy().sum(axis=2)
    want_dvs = dout.double().numpy().reshape(B, Hkv, G, T, d).sum(axis=(2, 3))
    assert np.abs(dvs - want_dvs).max() <= 1.5e-2 * max(1.0, np.abs(want_dvs).max())


def test_backward_deterministic_and_inputs_untouched(gqa):
    B, Hq, Hkv, T, d = 1, 4, 2, 300, 128
    q, k, v, dout = inputs(B, Hq, Hkv, T, d, "bf16", SEED + 3)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), dout.cuda()
    out, lse = gqa.attn_prefill_lse(qd, kd, vd)
    r1 = gqa.attn_backward(qd, kd, vd, out, dod, lse)
    r2 = gqa.attn_backward(qd, kd, vd, out, dod, lse)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(r1, r2))
    assert torch.equal(qd.cpu(), q) and torch.equal(dod.cpu(), dout)


def test_backward_rejects(gqa):
    lse = torch.zeros(1, 2, 8, device="cuda")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.zeros(1, 2, 8, 64, device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(gqa.GQAError):
        gqa.attn_backward(q, k, k, o, o, lse, workspace=small)


def test_full_size_backward_every_group(gqa):
    """The GQA prefill workload (B=2, 16 query / 8 K/V heads, T=4096, d=128, bf16) in the
    launch configuration the benchmark times; every (batch, K/V head) group checked in
    full against the oracle restricted to that group (max-abs and max-rel printed)."""
    cfg = si.GQA_T4096
    q, k, v = si.prefill_config_inputs(cfg)
    g = torch.Generator().manual_seed(cfg.seed + 100)
    dout = torch.randn(cfg.B, cfg.Hq, cfg.T, cfg.d, generator=g, dtype=torch.float32)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, lse = gqa.attn_prefill_lse(qd, kd, vd, scale=cfg.scale, causal=True)
    dq, dk, dv = gqa.attn_backward(qd, kd, vd, out, dout.cuda(), lse, scale=cfg.scale, causal=True)
    torch.cuda.synchronize()
    G = cfg.Hq // cfg.Hkv
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    stats = {n: [0.0, 0.0, 0.0] for n in ("dq", "dk", "dv")}  # max-abs, max |ref|, max-rel
    for b in range(cfg.B):
        print("backward oracle, batch %d" % b, flush=True)
        for gk in range(cfg.Hkv):
            hs = slice(gk * G, (gk + 1) * G)
            wq, wk, wv = bw.backward(q[b:b + 1, hs].double().numpy(), k[b:b + 1, gk:gk + 1].double().numpy(),
                                     v[b:b + 1, gk:gk + 1].double().numpy(), dout[b:b + 1, hs].double().numpy(),
                                     cfg.scale, True)
            for n, got, want in (("dq", dq[b:b + 1, hs], wq), ("dk", dk[b:b + 1, gk:gk + 1], wk),
                                 ("dv", dv[b:b + 1, gk:gk + 1], wv)):
                close(got, want)
                diff = np.abs(got.double().numpy() - want)
                st = stats[n]
                st[0] = max(st[0], float(diff.max()))
                st[1] = max(st[1], float(np.abs(want).max()))
                st[2] = max(st[2], float((diff / np.maximum(np.abs(want), 1.0)).max()))
    for n, (ma, mref, mrel) in stats.items():
        print("full-size %s: max-abs %.3g, max |ref| %.3g, max-abs / max(1, |ref|) %.3g" % (n, ma, mref, mrel))


GEN_CASES = [
    # B, Hq, Hkv, T, d, dtype, causal
    (2, 4, 2, 77, 64, "f32", True),
    (1, 3, 1, 50, 24, "f32", False),
    (1, 2, 2, 130, 128, "f32", True),
    (2, 4, 2, 100, 40, "bf16", True),
    (1, 2, 1, 33, 200, "f32", True),
    (1, 1, 1, 16, 8, "f32", True),
]


@pytest.mark.parametrize("case", GEN_CASES, ids=lambda c: "B%d_Hq%d_Hkv%d_T%d_d%d_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "causal" if c[6] else "full"))
def test_vector_backward_matches_oracle(gqa, case):
    B, Hq, Hkv, T, d, dtype, causal = case
    q, k, v, dout = inputs(B, Hq, Hkv, T, d, dtype, SEED + 11 * T + d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = d ** -0.5
    out, lse = gqa.attn_prefill_lse(qd, kd, vd, scale=scale, causal=causal)
    dq, dk, dv = gqa.attn_backward(qd, kd, vd, out, dout.cuda(), lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    wq, wk, wv = bw.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                             scale, causal)
    rel = 1e-4 if dtype == "f32" else 1.5e-2
    close(dq, wq, rel)
    close(dk, wk, rel)
    close(dv, wv, rel)


def test_vector_backward_single_head_workload(gqa):
    """The single-head fp32 workload (B=1, H=1, T=16, d=8, scale 1/sqrt(8)) through the
    forward with statistics and the vector-ALU backward."""
    cfg = si.SINGLE_HEAD_T16_F32
    q, k, v = si.prefill_config_inputs(cfg)
    g = torch.Generator().manual_seed(cfg.seed + 100)
    dout = torch.randn(cfg.B, cfg.Hq, cfg.T, cfg.d, generator=g, dtype=torch.float32)
    out, lse = gqa.attn_prefill_lse(q.cuda(), k.cuda(), v.cuda(), scale=cfg.scale, causal=True)
    grads = gqa.attn_backward(q.cuda(), k.cuda(), v.cuda(), out, dout.cuda(), lse, scale=cfg.scale)
    torch.cuda.synchronize()
    wants = bw.backward(q.double().numpy(), k.double().numpy(), v.double().numpy(), dout.double().numpy(),
                        cfg.scale, True)
    for got, want in zip(grads, wants):
        close(got, want, 1e-4)
