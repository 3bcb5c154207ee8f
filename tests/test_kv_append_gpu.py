"""KV-cache append with NeoX RoPE on K (attn_kv_append, attn_kv_append_paged) on the GPU
against the float64 oracle (oracle.kv_append).

The cache is written in its dtype, so the bar is the rounding of that dtype:

* V rows and unrotated K rows are a float32 -> cache-dtype conversion: bit-exact against
  torch's round-to-nearest-even conversion of the same values;
* rotated K: the kernel rotates in float32 (angles formed in float64) and rounds once to
  the cache dtype.  Each element must lie within one unit in the last place of the cache
  dtype of the exact float64 value, plus the float32 rotation error, bounded by
  4 * 2^-24 * (|k1| + |k2|) for the pair (k1, k2) it comes from;
* every row the call does not own keeps its bits.

Positions reach 32767 (the long decode history) so the angle's reduction is exercised; head dims
64, 80 (the BitNet-3B shape) and 128; float32 and bf16 caches; paged pools with blocks
in random order, and sequences whose metadata does not fit are left unwritten.
"""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from oracle import kv_append as ka

pytestmark = pytest.mark.gpu

SEED = si.SEED_BASE + 40


@pytest.fixture(scope="module")
def gqa():
    import grouped_query_attention_amd as m
    return m


def ulp(x, dtype):
    """Unit in the last place of |x| in the cache dtype (8 significant bits for bf16)."""
    bits = 8 if dtype == torch.bfloat16 else 24
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - (bits - 1))


def check_rotated(got, want, k_src, dtype):
    """got, want [..., d]; k_src [..., d] the unrotated float32 rows the values come from."""
    d = want.shape[-1]
    h = d // 2
    pair = np.abs(k_src[..., :h]) + np.abs(k_src[..., h:])
    bound = ulp(want, dtype) + 4 * 2.0 ** -24 * np.concatenate([pair, pair], axis=-1)
    err = np.abs(got - want)
    assert np.all(err <= bound), float((err / bound).max())


CASES = [
    # B, n, Hkv, d, L, start_pos, dtype, rope_base, factors
    (3, 5, 4, 128, 40, 30, torch.bfloat16, 10000.0, True),
    (2, 4, 8, 128, 32768, 32764, torch.bfloat16, 10000.0, False),
    (2, 1, 8, 128, 32768, 32767, torch.bfloat16, 500000.0, True),
    (1, 7, 2, 80, 100, 0, torch.bfloat16, 10000.0, False),
    (2, 3, 3, 64, 20, 17, torch.float32, 10000.0, True),
    (2, 2, 2, 64, 9000, 8999 - 1, torch.float32, 1000000.0, False),
    (2, 6, 4, 128, 16, 10, torch.bfloat16, 0.0, False),   # no rotation: plain copy
    (1, 1, 1, 8, 4, 3, torch.bfloat16, 10000.0, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_n%d_h%d_d%d_L%d_p%d_%s_base%g%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "bf16" if c[6] == torch.bfloat16 else "f32", c[7], "_ff" if c[8] else ""))
def test_append_matches_oracle(gqa, case):
    B, n, Hkv, d, L, sp, dt, base, use_ff = case
    k_new, v_new, kc, vc, ff = si.kv_append_inputs(B, n, Hkv, d, L, "bf16" if dt == torch.bfloat16 else "f32",
                                                   SEED + d + n)
    kc_d, vc_d = kc.cuda(), vc.cuda()
    gqa.attn_kv_append(k_new.cuda(), v_new.cuda(), kc_d, vc_d, sp, rope_base=base,
                       freq_factors=ff.cuda() if use_ff else None)
    torch.cuda.synchronize()
    kg, vg = kc_d.cpu(), vc_d.cpu()
    # untouched rows keep their bits
    keep = torch.cat([torch.arange(0, sp), torch.arange(sp + n, L)])
    assert torch.equal(kg[:, :, keep], kc[:, :, keep]) and torch.equal(vg[:, :, keep], vc[:, :, keep])
    # V: float32 -> cache dtype, bit-exact
    assert torch.equal(vg[:, :, sp:sp + n], v_new.transpose(1, 2).to(dt))
    if base == 0.0:
        assert torch.equal(kg[:, :, sp:sp + n], k_new.transpose(1, 2).to(dt))
        return
    kw, _ = ka.kv_append(kc.double().numpy(), vc.double().numpy(), k_new.double().numpy(),
                         v_new.double().numpy(), sp, rope_base=base,
                         freq_factors=ff.double().numpy() if use_ff else None)
    check_rotated(kg[:, :, sp:sp + n].double().numpy(), kw[:, :, sp:sp + n],
                  k_new.double().numpy().transpose(0, 2, 1, 3), dt)


def test_append_then_decode(gqa):
    """Append the new tokens with RoPE, then decode over the cache: equals the float64
    oracle's append followed by its cached decode (bf16 cache, so K goes through the
    same rounding on both sides: the oracle rounds its exact rotated rows to bf16)."""
    import oracle
    B, n, Hq, Hkv, d, L = 2, 4, 8, 2, 128, 300
    sp = L - n
    k_new, v_new, kc, vc, ff = si.kv_append_inputs(B, n, Hkv, d, L, "bf16", SEED + 1)
    q = si.decode_query(B, n, Hq, d, "bf16", SEED + 2)
    kc_d, vc_d = kc.cuda(), vc.cuda()
    gqa.attn_kv_append(k_new.cuda(), v_new.cuda(), kc_d, vc_d, sp, rope_base=10000.0, freq_factors=ff.cuda())
    out = gqa.attn_decode_cached(q.cuda(), kc_d, vc_d, sp)
    torch.cuda.synchronize()
    kw, vw = ka.kv_append(kc.double().numpy(), vc.double().numpy(), k_new.double().numpy(),
                          v_new.double().numpy(), sp, 10000.0, ff.double().numpy())
    kb = torch.from_numpy(kw).to(torch.bfloat16)  # the cache holds bf16 values
    vb = torch.from_numpy(vw).to(torch.bfloat16)
    want = oracle.decode_cached(q, kb, vb, sp)
    assert np.abs(out.cpu().double().numpy() - want).max() <= 1.5e-2


def test_full_size_prefill_append(gqa):
    """The benchmark's prefill-sized append: B=2, 4096 new tokens, 8 K/V heads, d=128, into
    a 4096-position bf16 cache, positions 0..4095; every element checked."""
    B, n, Hkv, d, L = 2, 4096, 8, 128, 4096
    k_new, v_new, kc, vc, ff = si.kv_append_inputs(B, n, Hkv, d, L, "bf16", SEED + 3)
    kc_d, vc_d = kc.cuda(), vc.cuda()
    gqa.attn_kv_append(k_new.cuda(), v_new.cuda(), kc_d, vc_d, 0, rope_base=10000.0)
    torch.cuda.synchronize()
    assert torch.equal(vc_d.cpu(), v_new.transpose(1, 2).to(torch.bfloat16))
    src = k_new.double().numpy().transpose(0, 2, 1, 3)
    want = ka.rope_neox(src, np.arange(n), 10000.0)
    check_rotated(kc_d.cpu().double().numpy(), want, src, torch.bfloat16)


def test_paged_append_matches_oracle(gqa):
    B, n, Hkv, d, bs = 4, 3, 2, 128, 16
    lens = [3, 40, 16, 100]
    max_blocks = 8
    table, nblk = si.paged_layout(lens, bs, max_blocks, SEED + 4, spare_blocks=3)
    g = torch.Generator().manual_seed(SEED + 5)
    kp = si.normal((nblk, Hkv, bs, d), g, "bf16")
    vp = si.normal((nblk, Hkv, bs, d), g, "bf16")
    k_new, v_new, _, _, ff = si.kv_append_inputs(B, n, Hkv, d, 1, "bf16", SEED + 6)
    lens_t = torch.tensor(lens, dtype=torch.int32)
    kp_d, vp_d = kp.cuda(), vp.cuda()
    gqa.attn_kv_append_paged(k_new.cuda(), v_new.cuda(), kp_d, vp_d, table.cuda(), lens_t.cuda(),
                             rope_base=10000.0, freq_factors=ff.cuda())
    torch.cuda.synchronize()
    kw, _ = ka.kv_append_paged(kp.double().numpy(), vp.double().numpy(), table.numpy(), lens,
                                k_new.double().numpy(), v_new.double().numpy(), 10000.0, ff.double().numpy())
    kg, vg = kp_d.cpu(), vp_d.cpu()
    written = np.zeros((nblk, bs), dtype=bool)
    tab = table.numpy()
    for b in range(B):
        for p in range(lens[b] - n, lens[b]):
            written[tab[b, p // bs], p % bs] = True
    for blk in range(nblk):
        for r in range(bs):
            if not written[blk, r]:
                assert torch.equal(kg[blk, :, r], kp[blk, :, r]) and torch.equal(vg[blk, :, r], vp[blk, :, r])
    # written rows: V exact, K within the rounding bound
    for b in range(B):
        for i, p in enumerate(range(lens[b] - n, lens[b])):
            blk, r = tab[b, p // bs], p % bs
            assert torch.equal(vg[blk, :, r], v_new[b, i].to(torch.bfloat16))
            src = k_new[b, i].double().numpy()
            check_rotated(kg[blk, :, r].double().numpy(), kw[blk, :, r], src, torch.bfloat16)


def test_paged_append_skips_bad_metadata(gqa):
    """A length below newTokens, a length beyond the table's reach and a -1 entry: those
    sequences are not written; the valid one is."""
    B, n, Hkv, d, bs, max_blocks = 4, 2, 1, 64, 16, 2
    nblk = 8
    table = torch.tensor([[0, 1], [2, 3], [4, -1], [6, 7]], dtype=torch.int32)
    lens = torch.tensor([1, 33, 20, 30], dtype=torch.int32)  # too short, beyond reach, -1 entry, valid
    g = torch.Generator().manual_seed(SEED + 7)
    kp = si.normal((nblk, Hkv, bs, d), g, "bf16")
    vp = si.normal((nblk, Hkv, bs, d), g, "bf16")
    k_new = si.normal((B, n, Hkv, d), g, "f32")
    v_new = si.normal((B, n, Hkv, d), g, "f32")
    kp_d, vp_d = kp.cuda(), vp.cuda()
    gqa.attn_kv_append_paged(k_new.cuda(), v_new.cuda(), kp_d, vp_d, table.cuda(), lens.cuda(), rope_base=0.0)
    torch.cuda.synchronize()
    kg, vg = kp_d.cpu(), vp_d.cpu()
    assert torch.equal(kg[:6], kp[:6]) and torch.equal(vg[:6], vp[:6])
    assert torch.equal(kg[7, :, 12:14], k_new[3].transpose(0, 1).to(torch.bfloat16))  # positions 28, 29
    assert torch.equal(kg[7, :, :12], kp[7, :, :12]) and torch.equal(kg[6], kp[6])


def test_append_deterministic_and_inputs_untouched(gqa):
    B, n, Hkv, d, L = 2, 3, 2, 128, 64
    k_new, v_new, kc, vc, ff = si.kv_append_inputs(B, n, Hkv, d, L, "bf16", SEED + 8)
    kn, vn = k_new.cuda(), v_new.cuda()
    outs = []
    for _ in range(2):
        kc_d, vc_d = kc.cuda(), vc.cuda()
        gqa.attn_kv_append(kn, vn, kc_d, vc_d, 50, rope_base=10000.0, freq_factors=ff.cuda())
        outs.append((kc_d.cpu(), vc_d.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert torch.equal(kn.cpu(), k_new) and torch.equal(vn.cpu(), v_new)
