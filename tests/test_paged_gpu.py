"""Paged (block-table) decode on the GPU against the float64 oracle.

attn_decode_paged reads each sequence's K/V history out of a fragmented block pool
through a block table (makarna's CausalAttentionPackedBlocks; the "paged decode
attention" of Riftco's "Algorithm and cache boundaries").  Checked here:

* element-wise parity with oracle.decode_paged on ragged lengths (length = newTokens,
  block boundaries, several key chunks), block sizes 16..256 including 48, head dims
  16..128, G = 1..8 and newTokens 1..16; pool slots no sequence owns hold NaN, so any
  read of them would show;
* bitwise equality with attn_decode_cached on the same history (same kernels, same
  split plan, only the addressing differs);
* device-side metadata errors (length out of range, table entry outside the pool)
  turn that sequence's rows into NaN and leave the others exact;
* shared blocks, determinism.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu

TOL = 1.5e-2  # bf16 inputs, fp32 accumulation


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


CASES = [
    # B, n, Hq, Hkv, d, block_size, lens, max_blocks
    (3, 1, 8, 2, 128, 16, [1, 100, 1000], 64),
    (2, 4, 16, 4, 64, 32, [4, 517], 20),
    (2, 5, 16, 4, 128, 48, [700, 300], 16),
    (1, 3, 4, 4, 80, 256, [2000], 8),
    (4, 2, 32, 8, 128, 64, [64, 65, 128, 3000], 50),
    (1, 1, 8, 1, 128, 16, [5000], 400),
    (2, 16, 8, 8, 32, 16, [16, 40], 4),
    (1, 2, 2, 1, 16, 16, [33], 3),
    (3, 1, 32, 8, 96, 128, [129, 1, 255], 2),
]


def case_id(c):
    B, n, Hq, Hkv, d, bs, lens, mb = c
    return "B%dn%dHq%dHkv%dd%dbs%d-L%s" % (B, n, Hq, Hkv, d, bs, "_".join(map(str, lens)))


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_paged_decode_matches_oracle(gqa, case):
    B, n, Hq, Hkv, d, bs, lens, mb = case
    seed = 4242 + sum(lens)
    q, kp, vp, table, sl = si.paged_decode_inputs(B, n, Hq, Hkv, d, bs, lens, mb, "bf16", seed,
                                                  spare_blocks=3)
    print("paged", case_id(case), flush=True)
    out = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), sl.cuda())
    torch.cuda.synchronize()
    want = oracle.decode_paged(q, kp, vp, table, lens, bs)
    err = float(np.abs(out.cpu().double().numpy() - want).max())
    print("max-abs error %.3g" % err)
    assert err <= TOL, err


@pytest.mark.parametrize("n", [1, 4])
def test_paged_bitwise_equals_contiguous(gqa, n):
    B, Hq, Hkv, d, L, bs = 3, 16, 4, 128, 3000, 96  # 3000 is not a multiple of 96
    mb = -(-L // bs)
    seed = 777 + n
    q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, "bf16", seed)
    table, nb = si.paged_layout([L] * B, bs, mb, seed, spare_blocks=5)
    kp = torch.full((nb, Hkv, bs, d), float("nan"), dtype=torch.bfloat16)
    vp = torch.full_like(kp, float("nan"))
    for b in range(B):
        si.scatter_history(kp, table[b], kc[b], bs)
        si.scatter_history(vp, table[b], vc[b], bs)
    sl = torch.full((B,), L, dtype=torch.int32)
    # the contiguous call sees the same history with the cache padded to the table's
    # reach (rows past the history are never read)
    pad = mb * bs - L
    kcp = torch.cat([kc, torch.full((B, Hkv, pad, d), float("nan"), dtype=kc.dtype)], dim=2)
    vcp = torch.cat([vc, torch.full((B, Hkv, pad, d), float("nan"), dtype=vc.dtype)], dim=2)
    print("paged vs contiguous n=%d" % n, flush=True)
    a = gqa.attn_decode_cached(q.cuda(), kcp.cuda(), vcp.cuda(), L - n)
    p = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), sl.cuda())
    torch.cuda.synchronize()
    assert not torch.isnan(a).any()
    assert torch.equal(a, p)


def test_paged_bad_metadata_poisons_only_that_sequence(gqa):
    B, n, Hq, Hkv, d, bs, mb = 5, 2, 8, 2, 64, 16, 10
    lens = [100, 50, 60, 70, 80]
    q, kp, vp, table, sl = si.paged_decode_inputs(B, n, Hq, Hkv, d, bs, lens, mb, "bf16", 99)
    want = oracle.decode_paged(q, kp, vp, table, lens, bs)
    nb = kp.shape[0]
    bad_lens = sl.clone()
    bad_lens[1] = n - 1          # shorter than the new tokens
    bad_lens[2] = mb * bs + 1    # longer than the table can describe
    bad_table = table.clone()
    bad_table[3, 2] = -1         # a needed entry below the pool
    bad_table[4, 4] = nb         # a needed entry past the pool
    print("paged bad metadata", flush=True)
    out = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), bad_table.cuda(), bad_lens.cuda())
    torch.cuda.synchronize()
    out = out.cpu()
    for b in (1, 2, 3, 4):
        assert torch.isnan(out[b]).all(), b
    err = float(np.abs(out[0].double().numpy() - want[0]).max())
    assert err <= TOL, err


def test_paged_shared_blocks_and_determinism(gqa):
    B, n, Hq, Hkv, d, bs, mb = 2, 3, 16, 4, 128, 32, 40
    q, kp, vp, table, sl = si.paged_decode_inputs(1, n, Hq, Hkv, d, bs, [1200], mb, "bf16", 5)
    q2 = torch.cat([q, q])
    t2 = torch.cat([table, table])
    s2 = torch.cat([sl, sl])
    print("paged shared blocks", flush=True)
    o1 = gqa.attn_decode_paged(q2.cuda(), kp.cuda(), vp.cuda(), t2.cuda(), s2.cuda())
    o2 = gqa.attn_decode_paged(q2.cuda(), kp.cuda(), vp.cuda(), t2.cuda(), s2.cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1[0], o1[1])
    assert torch.equal(o1, o2)
    # a shorter sequence over the same blocks: the prefix of the history
    s3 = torch.tensor([1200, 700], dtype=torch.int32)
    o3 = gqa.attn_decode_paged(q2.cuda(), kp.cuda(), vp.cuda(), t2.cuda(), s3.cuda())
    torch.cuda.synchronize()
    want = oracle.decode_paged(q2, kp, vp, t2, [1200, 700], bs)
    assert float(np.abs(o3.cpu().double().numpy() - want).max()) <= TOL


def test_paged_inputs_not_modified(gqa):
    q, kp, vp, table, sl = si.paged_decode_inputs(2, 2, 8, 2, 64, 16, [90, 33], 8, "bf16", 12,
                                                  fill=0.0)
    args = [t.cuda() for t in (q, kp, vp, table, sl)]
    before = [t.clone() for t in args]
    gqa.attn_decode_paged(*args)
    torch.cuda.synchronize()
    for a, b in zip(args, before):
        assert torch.equal(a, b)
