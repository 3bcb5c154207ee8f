"""Decode over token-major blocks (attn_decode_blocks) on the GPU against the float64 oracle.

attn_decode_blocks is makarna's CausalAttentionBlocks: the history lives in views laid
out token by token ([tokenWithinBlock][kvHead][headDim]), here the blocks a block table
names.  Checked here:

* element-wise parity with oracle.decode_blocks (which walks the views as the page does)
  on ragged lengths, block sizes 16..256, head dims 16..128, G = 1..8 and newTokens
  1..16, with every pool slot no sequence owns set to NaN;
* bitwise equality with attn_decode_paged on the same blocks stored head-major (same
  kernels and split plan, only the row addressing differs);
* device-side metadata errors turn that sequence's rows into NaN and leave the others
  exact, as in attn_decode_paged.
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
    (2, 16, 8, 8, 32, 16, [16, 40], 4),
    (1, 2, 2, 1, 16, 16, [33], 3),
    (3, 1, 32, 8, 96, 128, [129, 1, 255], 2),
]


def case_id(c):
    B, n, Hq, Hkv, d, bs, lens, mb = c
    return "B%dn%dHq%dHkv%dd%dbs%d-L%s" % (B, n, Hq, Hkv, d, bs, "_".join(map(str, lens)))


def token_major(pool):
    """[num_blocks, Hkv, bs, d] -> [num_blocks, bs, Hkv, d], the same values."""
    return pool.permute(0, 2, 1, 3).contiguous()


@pytest.mark.parametrize("case", CASES, ids=case_id)
def test_blocks_decode_matches_oracle(gqa, case):
    B, n, Hq, Hkv, d, bs, lens, mb = case
    seed = 5151 + sum(lens)
    q, kp, vp, table, sl = si.paged_decode_inputs(B, n, Hq, Hkv, d, bs, lens, mb, "bf16", seed,
                                                  spare_blocks=3)
    kt, vt = token_major(kp), token_major(vp)
    print("blocks", case_id(case), flush=True)
    out = gqa.attn_decode_blocks(q.cuda(), kt.cuda(), vt.cuda(), table.cuda(), sl.cuda())
    torch.cuda.synchronize()
    want = oracle.decode_blocks(q, kt, vt, table, lens, bs)
    err = float(np.abs(out.cpu().double().numpy() - want).max())
    print("max-abs error %.3g" % err)
    assert err <= TOL, err


@pytest.mark.parametrize("n", [1, 4])
def test_blocks_bitwise_equals_paged(gqa, n):
    B, Hq, Hkv, d, bs, mb = 3, 16, 4, 128, 64, 60
    lens = [3000, 1777, 64]
    q, kp, vp, table, sl = si.paged_decode_inputs(B, n, Hq, Hkv, d, bs, lens, mb, "bf16", 31 + n,
                                                  spare_blocks=4)
    print("blocks vs paged n=%d" % n, flush=True)
    p = gqa.attn_decode_paged(q.cuda(), kp.cuda(), vp.cuda(), table.cuda(), sl.cuda())
    t = gqa.attn_decode_blocks(q.cuda(), token_major(kp).cuda(), token_major(vp).cuda(), table.cuda(),
                               sl.cuda())
    torch.cuda.synchronize()
    assert not torch.isnan(p).any()
    assert torch.equal(p, t)


def test_blocks_bad_metadata_poisons_only_that_sequence(gqa):
    B, n, Hq, Hkv, d, bs, mb = 4, 2, 8, 2, 64, 16, 10
    lens = [100, 50, 60, 70]
    q, kp, vp, table, sl = si.paged_decode_inputs(B, n, Hq, Hkv, d, bs, lens, mb, "bf16", 77)
    kt, vt = token_major(kp), token_major(vp)
    want = oracle.decode_blocks(q, kt, vt, table, lens, bs)
    bad_lens = sl.clone()
    bad_lens[1] = mb * bs + 1    # longer than the table can describe
    bad_table = table.clone()
    bad_table[2, 1] = -1         # a needed entry below the pool
    bad_table[3, 3] = kp.shape[0]  # a needed entry past the pool
    print("blocks bad metadata", flush=True)
    out = gqa.attn_decode_blocks(q.cuda(), kt.cuda(), vt.cuda(), bad_table.cuda(), bad_lens.cuda())
    torch.cuda.synchronize()
    out = out.cpu()
    for b in (1, 2, 3):
        assert torch.isnan(out[b]).all(), b
    err = float(np.abs(out[0].double().numpy() - want[0]).max())
    assert err <= TOL, err


def test_blocks_host_errors(gqa):
    q, kp, vp, table, sl = si.paged_decode_inputs(1, 1, 4, 2, 64, 16, [40], 4, "bf16", 3)
    kt, vt = token_major(kp).cuda(), token_major(vp).cuda()
    with pytest.raises(gqa.GQAError):  # fp32 pools are not supported
        gqa.attn_decode_blocks(q.float().cuda(), kt.float(), vt.float(), table.cuda(), sl.cuda())
    kt8 = token_major(kp[:, :, :8]).cuda()  # block size 8: not a multiple of 16
    with pytest.raises(gqa.GQAError):
        gqa.attn_decode_blocks(q.cuda(), kt8, kt8, table.cuda(), sl.cuda())
