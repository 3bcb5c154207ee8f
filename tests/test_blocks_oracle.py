"""Pins of the token-major views oracle (oracle.decode_views, oracle.decode_blocks) on the CPU.

makarna's CausalAttentionBlocks attends over a list of views, each holding the keys of
positions Start .. Start+Length-1 token by token ([t, Hkv*headDim]); new token i at
position startPos+i sees the keys below startPos+i+1, whatever view they are in.  The
pins check the oracle against:

1. a closed form: with q = 0 every visible key weighs the same, so each output row is
   the plain mean of the V rows its token sees, counted here from a position -> row map
   (views with gaps, unequal lengths, listed out of order, and a token that sees none);
2. the contiguous-cache C oracle, on views cut from one history at uneven points;
3. the paged oracle, on the same blocks stored head-major instead of token-major, with
   every slot no sequence owns set to NaN.

A limit off by one, a wrong KV head for a query head, or a transposed block fails one of
them.
"""
import numpy as np
import pytest

import oracle


def test_zero_query_gives_the_mean_of_the_visible_rows():
    rng = np.random.default_rng(11)
    Hq, Hkv, d, n, start_pos = 6, 3, 4, 3, 9
    spans = [(10, 2), (0, 4), (6, 3), (20, 5), (4, 0)]  # (start, length); 4..5 is a gap
    rows = {}
    views = []
    for start, length in spans:
        k = rng.standard_normal((length, Hkv * d))
        v = rng.standard_normal((length, Hkv * d))
        for t in range(length):
            rows[start + t] = v[t].reshape(Hkv, d)
        views.append((start, k, v))
    q = np.zeros((n, Hq, d))
    got = oracle.decode_views(q, views, start_pos, Hkv)
    for i in range(n):
        seen = sorted(p for p in rows if p < start_pos + i + 1)
        for h in range(Hq):
            want = np.mean([rows[p][h // (Hq // Hkv)] for p in seen], axis=0)
            np.testing.assert_allclose(got[i, h], want, rtol=0, atol=1e-12)
    # positions 0..3, 6..8 for token 0; 10 joins at token 1, 11 at token 2
    assert [len([p for p in rows if p < start_pos + i + 1]) for i in range(n)] == [7, 8, 9]


def test_a_token_that_sees_no_key_is_zero():
    rng = np.random.default_rng(3)
    views = [(5, rng.standard_normal((4, 8)), rng.standard_normal((4, 8)))]
    got = oracle.decode_views(rng.standard_normal((2, 2, 4)), views, 3, 2)
    assert np.all(got[0] == 0) and np.all(got[1] == 0)


@pytest.mark.parametrize("L,n,cuts", [(23, 1, [5, 6, 17]), (40, 4, [16, 32]), (9, 3, [1, 2, 8])])
def test_views_of_one_history_match_the_cached_decode(L, n, cuts):
    rng = np.random.default_rng(L)
    Hq, Hkv, d = 4, 2, 8
    kh = rng.standard_normal((Hkv, L, d))
    vh = rng.standard_normal((Hkv, L, d))
    q = rng.standard_normal((n, Hq, d))
    edges = [0] + cuts + [L]
    views = [(a, kh[:, a:b_, :].transpose(1, 0, 2).reshape(b_ - a, Hkv * d),
              vh[:, a:b_, :].transpose(1, 0, 2).reshape(b_ - a, Hkv * d))
             for a, b_ in zip(edges[:-1], edges[1:])][::-1]
    got = oracle.decode_views(q, views, L - n, Hkv)
    want = oracle.decode_cached(q[None], kh[None], vh[None], L - n)[0]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_token_major_blocks_match_the_paged_oracle():
    rng = np.random.default_rng(5)
    B, n, Hq, Hkv, d, bs = 3, 2, 4, 2, 8, 4
    lens = [2, 9, 13]
    need = [-(-L // bs) for L in lens]
    num_blocks = sum(need) + 2
    perm = rng.permutation(num_blocks)
    table = np.full((B, 5), -1, dtype=np.int64)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    kpool = np.full((num_blocks, bs, Hkv, d), np.nan)
    vpool = np.full((num_blocks, bs, Hkv, d), np.nan)
    for b, L in enumerate(lens):
        for p in range(L):
            kpool[table[b, p // bs], p % bs] = rng.standard_normal((Hkv, d))
            vpool[table[b, p // bs], p % bs] = rng.standard_normal((Hkv, d))
    q = rng.standard_normal((B, n, Hq, d))
    got = oracle.decode_blocks(q, kpool, vpool, table, lens, bs)
    assert np.all(np.isfinite(got))
    want = oracle.decode_paged(q, kpool.transpose(0, 2, 1, 3), vpool.transpose(0, 2, 1, 3), table, lens, bs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
