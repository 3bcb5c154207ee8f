"""attn_decode_cached_noalloc (split-KV partials in the library's fixed device scratch,
no allocation) against attn_decode_cached with a caller workspace: the same kernels and
split plan, so the outputs must be bitwise equal, and both meet the oracle at the bf16
gate.  Two calls in a row on the same scratch, the second with a smaller shape, then an
fp32 call (which needs no scratch)."""
import os

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si

pytestmark = pytest.mark.gpu


def threads():
    return max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


SHAPES = [
    # B, n, Hq, Hkv, L, d, dtype: the first needs ~17 MB of partials, the second less
    (8, 4, 32, 8, 32768, 128, "bf16"),
    (2, 1, 8, 2, 1000, 64, "bf16"),
    (2, 3, 8, 2, 700, 128, "f32"),
]


def test_noalloc_equals_workspace_decode(gqa):
    for i, (B, n, Hq, Hkv, L, d, dtype) in enumerate(SHAPES):
        print("noalloc call %d: B%d n%d Hq%d Hkv%d L%d d%d %s" % (i, B, n, Hq, Hkv, L, d, dtype), flush=True)
        q, kc, vc = si.decode_inputs(B, n, Hq, Hkv, L, d, dtype, si.SEED_BASE + 900 + i)
        qd, kd, vd = q.cuda(), kc.cuda(), vc.cuda()
        need = gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d, gqa.GQA_BF16 if dtype == "bf16" else gqa.GQA_F32)
        assert need <= gqa.GQA_NOALLOC_SCRATCH_BYTES
        ref = gqa.attn_decode_cached(qd, kd, vd, L - n)
        out = torch.full((B, n, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        gqa.attn_decode_cached_noalloc(qd, kd, vd, L - n, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        want = oracle.decode_cached(q, kc, vc, L - n, nthreads=threads())
        err = float(np.abs(out.cpu().double().numpy() - want).max())
        print("  max-abs vs oracle %.3g" % err)
        assert err <= (1.5e-2 if dtype == "bf16" else 1e-4), (i, err)


def test_noalloc_rejects_shapes_beyond_the_scratch(gqa):
    # 64 sequences, 32 query heads, 64 new tokens over a 32768-position history: the
    # partials exceed the fixed scratch; rejected before anything is enqueued
    B, n, Hq, Hkv, L, d = 64, 64, 32, 8, 32768, 128
    assert gqa.attn_decode_workspace_bytes(B, n, L, Hq, Hkv, d) > gqa.GQA_NOALLOC_SCRATCH_BYTES
    fake = 0x10000
    rc = gqa.lib.attn_decode_cached_noalloc(fake, fake, fake, fake, n, L, L - n, Hq, Hkv, d, B, gqa.GQA_BF16, None)
    assert rc == gqa.GQA_ESCRATCH
