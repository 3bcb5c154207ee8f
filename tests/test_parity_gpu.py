"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Tolerances (max-abs over every output element, fp32 output):
  fp32 inputs 1e-4; bf16 inputs 1.5e-2 (bf16 operands, fp32 accumulation).
Both kernels (generic vector-ALU and bf16 matrix-core) are checked where they apply.
"""
import math

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


def maxerr(got, want):
    return float(np.abs(got.detach().cpu().double().numpy() - want).max())


def run_prefill(gqa, q, k, v, scale, causal, algo):
    out = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), scale=scale, causal=causal, algo=algo)
    torch.cuda.synchronize()
    return out


ALGOS = {"generic": 1, "mfma": 2, "split": 3}


def covers(gqa, dtype, d, algo, Hq=1, Hkv=1):
    # a zero-size call with an explicit kernel request reports whether it covers the shape
    code = gqa.GQA_BF16 if dtype == "bf16" else gqa.GQA_F32
    return gqa.lib.attn_prefill_ex(None, None, None, None, 0, Hq, Hkv, 1, d, 1.0, 1, code, algo, None) == 0


def mfma_covers(gqa, dtype, d, Hq=1, Hkv=1):
    return covers(gqa, dtype, d, ALGOS["mfma"], Hq, Hkv)


def algos_for(dtype, d, Hq=1, Hkv=1):
    """Every kernel that covers the shape: the vector kernel, the matrix-core kernel
    (one workgroup per q-tile) and the split-key matrix-core kernel."""
    import grouped_query_attention_amd as gqa
    a = ["generic"]
    for name in ("mfma", "split"):
        if covers(gqa, dtype, d, ALGOS[name], Hq, Hkv):
            a.append(name)
    return a


# --------------------------------------------------------------- worked example
def test_worked_example_prefill_and_decode(gqa):
    """Multi-query attention primer, section 2.1 Tiny example -> 2.0."""
    q = torch.zeros(1, 1, 3, 2)
    q[0, 0, 2] = torch.tensor([1.0, 0.0])
    k = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).reshape(1, 1, 3, 2)
    v = torch.tensor([[1.0, 0.0], [2.0, 0.0], [3.0, 0.0]]).reshape(1, 1, 3, 2)
    out = run_prefill(gqa, q, k, v, 1.0, True, ALGOS["generic"])
    assert abs(out[0, 0, 2, 0].item() - 2.0) < 1e-6 and out[0, 0, 2, 1].item() == 0.0
    qd = torch.tensor([math.sqrt(2.0), 0.0]).reshape(1, 1, 1, 2)
    outd = gqa.attn_decode_cached(qd.cuda(), k.cuda(), v.cuda(), 2)
    torch.cuda.synchronize()
    assert abs(outd[0, 0, 0, 0].item() - 2.0) < 1e-6


# ------------------------------------------------------------ small workloads
@pytest.mark.parametrize("cfg", [si.SINGLE_HEAD_T16_F32, si.MHA_T512_F32, si.MHA_T512_BF16], ids=lambda c: c.name)
def test_small_workloads(gqa, cfg):
    q, k, v = si.prefill_config_inputs(cfg)
    want = oracle.prefill(q, k, v, cfg.scale, True)
    for algo in algos_for(cfg.dtype, cfg.d):
        got = run_prefill(gqa, q, k, v, cfg.scale, True, ALGOS[algo])
        err = maxerr(got, want)
        print("%s %s maxerr %.3g" % (cfg.name, algo, err))
        assert err <= TOL[cfg.dtype], (algo, err)


RAGGED = [
    # B, Hq, Hkv, T, d, causal
    (1, 1, 1, 1, 8, True),
    (2, 4, 2, 37, 16, True),
    (1, 6, 3, 129, 64, True),
    (2, 8, 2, 200, 80, True),
    (1, 2, 1, 257, 128, True),
    (1, 4, 4, 96, 128, False),
    (2, 3, 1, 70, 1, True),
    (1, 2, 2, 45, 3, False),
    (1, 4, 2, 65, 200, True),
    (1, 2, 1, 33, 256, True),
    (3, 8, 8, 300, 96, True),
    (1, 16, 2, 190, 32, True),
    (2, 4, 2, 300, 64, False),   # full attention over several 128-row workgroup tiles
    (1, 2, 2, 1, 32, True),      # one row: a workgroup of padding rows
    (1, 4, 1, 128, 96, True),    # exactly one 128-row tile
    (1, 2, 1, 1000, 128, True),  # many key tiles, ragged end
    (2, 8, 4, 700, 64, True),    # split-key kernel with 4 splits per slice
    (2, 12, 12, 900, 32, True),  # split-key kernel with 2 splits per slice
    (1, 4, 2, 230, 112, True),   # fp32: padded head dims with head pairs at D = 128
    (1, 6, 2, 300, 128, True),   # group of 3: one head per workgroup
    (1, 8, 2, 333, 128, True),   # group of 4: two head pairs share each K/V tile
    (2, 16, 2, 257, 128, True),  # group of 8
    (1, 10, 2, 150, 48, True),   # group of 5, head dim 16 mod 32
    (2, 5, 1, 66, 112, False),   # odd head count sharing one K/V head, full attention
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", RAGGED, ids=lambda s: "B%dHq%dHkv%dT%dd%d%s" % (s[0], s[1], s[2], s[3], s[4],
                                                                                   "c" if s[5] else "n"))
def test_ragged_prefill(gqa, shape, dtype):
    B, Hq, Hkv, T, d, causal = shape
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=hash(shape) % 100000)
    scale = 1 / math.sqrt(d)
    want = oracle.prefill(q, k, v, scale, causal)
    for algo in algos_for(dtype, d):
        got = run_prefill(gqa, q, k, v, scale, causal, ALGOS[algo])
        err = maxerr(got, want)
        assert err <= TOL[dtype], (algo, err)


DECODE = [
    # B, n, Hq, Hkv, L, d
    (1, 1, 4, 1, 1, 64),
    (2, 1, 8, 2, 300, 128),
    (2, 4, 32, 8, 1000, 128),
    (3, 3, 6, 3, 517, 64),
    (1, 2, 4, 4, 4099, 80),
    (2, 1, 16, 1, 2049, 128),
    (1, 5, 2, 1, 77, 24),
    (1, 4, 16, 2, 300, 128),   # 32 query columns per group: two MFMA column blocks
    (2, 5, 16, 4, 2000, 64),   # 20 columns per group, a ragged second block
    (1, 40, 2, 1, 100, 64),    # new tokens span several 32-key chunks: all-masked partials
    (1, 33, 4, 1, 65, 128),    # every key is new; chunks smaller than the token span
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", DECODE, ids=lambda s: "B%dn%dHq%dHkv%dL%dd%d" % s)
def test_ragged_decode(gqa, shape, dtype):
    B, n, Hq, Hkv, L, d = shape
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dtype, seed=hash(shape) % 100000)
    want = oracle.decode_cached(q, kc, vc, L - n)
    got = gqa.attn_decode_cached(q.cuda(), kc.cuda(), vc.cuda(), L - n)
    torch.cuda.synchronize()
    err = maxerr(got, want)
    assert err <= TOL[dtype], err


def test_decode_start_pos_inside_cache(gqa):
    """New tokens need not be the last cache rows: keys after startPos+i are ignored."""
    B, n, Hq, Hkv, L, d = 2, 3, 8, 2, 700, 128
    for dtype in ("f32", "bf16"):
        q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dtype, seed=77)
        sp = 401
        want = oracle.decode_cached(q, kc[:, :, :sp + n], vc[:, :, :sp + n], sp)
        got = gqa.attn_decode_cached(q.cuda(), kc.cuda(), vc.cuda(), sp)
        torch.cuda.synchronize()
        assert maxerr(got, want) <= TOL[dtype]


# -------------------------------------------------------------- invariants
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128), ("bf16", 80)])
def test_rows_sum_to_one(gqa, dtype, d):
    """V == 1 everywhere -> every output is 1 (probabilities sum to one)."""
    B, Hq, Hkv, T = 2, 4, 2, 300
    q, k, _ = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=5)
    v = torch.ones_like(k)
    for algo in algos_for(dtype, d):
        got = run_prefill(gqa, q, k, v, 1 / math.sqrt(d), True, ALGOS[algo])
        # out = (sum_j p_j * 1) / (sum_j p_j); a kernel may form the two sums in different
        # orders (the fp32 matrix-core kernel sums the numerator inside the MFMA and the
        # normalizer per lane).  A sum of T positive fp32 terms is within (T-1)*2^-24 of
        # the exact one, relatively, so the quotient is within 2*T*2^-24 of 1.
        tol = 2 * T * 2.0 ** -24 if dtype == "f32" else 1e-2
        assert float((got - 1).abs().max()) <= tol, algo


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("bf16", 128)])
def test_future_keys_get_exactly_zero(gqa, dtype, d):
    """V rows are one-hot in the key index (T <= d): output component j of row i is
    exactly 0.0 for every future key j > i."""
    B, Hq, Hkv, T = 1, 2, 1, d
    q, k, _ = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=6)
    v = torch.eye(T, d).reshape(1, 1, T, d).repeat(B, Hkv, 1, 1).to(q.dtype)
    for algo in algos_for(dtype, d):
        got = run_prefill(gqa, q, k, v, 1 / math.sqrt(d), True, ALGOS[algo]).cpu()
        fut = torch.triu(torch.ones(T, d, dtype=torch.bool), diagonal=1)
        assert torch.all(got[..., fut] == 0.0), algo
        assert torch.all(got[..., ~fut] > 0.0), algo


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 80)])
def test_causality_bitwise(gqa, dtype, d):
    """Changing tokens after position t leaves rows <= t bit-for-bit unchanged."""
    B, Hq, Hkv, T = 1, 4, 2, 260
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=7)
    for algo in algos_for(dtype, d):
        base = run_prefill(gqa, q, k, v, 1 / math.sqrt(d), True, ALGOS[algo]).cpu()
        for t in (0, 63, 64, 150):
            q2, k2, v2 = q.clone(), k.clone(), v.clone()
            q2[:, :, t + 1:] = q2[:, :, t + 1:] * 3 + 1
            k2[:, :, t + 1:] = -k2[:, :, t + 1:]
            v2[:, :, t + 1:] = v2[:, :, t + 1:] * 5
            got = run_prefill(gqa, q2, k2, v2, 1 / math.sqrt(d), True, ALGOS[algo]).cpu()
            assert torch.equal(got[:, :, :t + 1], base[:, :, :t + 1]), (algo, t)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_gqa_equals_mha(gqa, dtype, d):
    B, Hq, Hkv, T = 2, 8, 2, 200
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=8)
    G = Hq // Hkv
    for algo in algos_for(dtype, d):
        a = run_prefill(gqa, q, k, v, 1 / math.sqrt(d), True, ALGOS[algo])
        b = run_prefill(gqa, q, k.repeat_interleave(G, 1).contiguous(), v.repeat_interleave(G, 1).contiguous(),
                        1 / math.sqrt(d), True, ALGOS[algo])
        assert float((a - b).abs().max()) <= (1e-6 if dtype == "f32" else 1e-3), algo


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_decode_equals_prefill_rows(gqa, dtype, d):
    B, Hq, Hkv, T = 2, 8, 2, 333
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, dtype, seed=9)
    full = run_prefill(gqa, q, k, v, 1 / math.sqrt(d), True, 0)
    for n in (1, 4):
        qd = q[:, :, T - n:].transpose(1, 2).contiguous()  # [B, n, Hq, d]
        dec = gqa.attn_decode_cached(qd.cuda(), k.cuda(), v.cuda(), T - n)
        torch.cuda.synchronize()
        ref = full[:, :, T - n:].transpose(1, 2)
        assert float((dec - ref).abs().max()) <= (1e-5 if dtype == "f32" else 5e-3), n


def test_inputs_not_modified(gqa):
    B, Hq, Hkv, T, d = 1, 4, 2, 100, 128
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, "bf16", seed=11)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    gqa.attn_prefill(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k) and torch.equal(vd.cpu(), v)


def test_output_guard_bands_untouched(gqa):
    """Writes stay inside out: sentinel regions before and after are unchanged."""
    B, Hq, Hkv, T, d = 2, 4, 2, 77, 80
    q, k, v = si.prefill_inputs(B, Hq, Hkv, T, d, "bf16", seed=12)
    n = B * Hq * T * d
    pad = 4096
    buf = torch.full((n + 2 * pad,), 7.25, dtype=torch.float32, device="cuda")
    out = buf[pad:pad + n].view(B, Hq, T, d)
    for algo in algos_for("bf16", d):
        gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda(), out=out, algo=ALGOS[algo])
        torch.cuda.synchronize()
        assert torch.all(buf[:pad] == 7.25) and torch.all(buf[pad + n:] == 7.25), algo


def test_deterministic(gqa):
    q, k, v = si.prefill_inputs(2, 8, 4, 513, 128, "bf16", seed=13)
    a = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda())
    b = gqa.attn_prefill(q.cuda(), k.cuda(), v.cuda())
    torch.cuda.synchronize()
    assert torch.equal(a, b)
