"""Pins of the paged-decode oracle (oracle.decode_paged / oracle.gather_paged) on the CPU.

The paged decode of makarna's CausalAttentionPackedBlocks is the cached decode of each
sequence over the history its blocks hold: logical block i is the view with Start =
i * block_size and Length = min(block_size, seq_len - Start), stored head-major inside
the block ([kvHead][tokenWithinBlock][headDim]).  The pins below check the oracle
against (1) the contiguous-cache oracle on a history this file scatters into a pool
element by element, (2) a direct loop over the views in the pages' order with a
materialized softmax, written here in plain Python, and (3) invariances of the table
(ignored entries, shared blocks).  Planted mistakes in the gather must fail them.
"""
import math

import numpy as np
import pytest

import oracle


def scatter_elementwise(hists, table, num_blocks, block_size):
    """hists[b]: [Hkv, L_b, d] -> pool [num_blocks, Hkv, block_size, d]; position p of
    sequence b goes to block table[b][p // block_size], slot p % block_size.  Unowned
    slots hold NaN (the oracle must never read them)."""
    Hkv, _, d = hists[0].shape
    pool = np.full((num_blocks, Hkv, block_size, d), np.nan)
    for b, hist in enumerate(hists):
        for p in range(hist.shape[1]):
            blk = table[b][p // block_size]
            for h in range(Hkv):
                pool[blk, h, p % block_size, :] = hist[h, p, :]
    return pool


def make_case(rng, B, n, Hq, Hkv, d, block_size, lens, max_blocks, spare=2):
    need = [-(-L // block_size) for L in lens]
    num_blocks = sum(need) + spare
    perm = rng.permutation(num_blocks)
    table = np.full((B, max_blocks), -1, dtype=np.int64)
    at = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[at:at + nb]
        at += nb
    q = rng.standard_normal((B, n, Hq, d))
    kh = [rng.standard_normal((Hkv, L, d)) for L in lens]
    vh = [rng.standard_normal((Hkv, L, d)) for L in lens]
    kpool = scatter_elementwise(kh, table, num_blocks, block_size)
    vpool = scatter_elementwise(vh, table, num_blocks, block_size)
    return q, kh, vh, kpool, vpool, table


CASES = [
    # B, n, Hq, Hkv, d, block_size, lens, max_blocks
    (3, 1, 4, 2, 8, 4, [1, 7, 12], 4),
    (2, 3, 6, 2, 5, 3, [3, 10], 5),
    (2, 2, 2, 1, 4, 5, [5, 6], 3),
    (1, 4, 3, 3, 6, 16, [40], 3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d-n%d-bs%d" % (c[0], c[1], c[5]))
def test_paged_equals_contiguous_per_sequence(case):
    B, n, Hq, Hkv, d, bs, lens, mb = case
    rng = np.random.default_rng(7)
    q, kh, vh, kpool, vpool, table = make_case(rng, B, n, Hq, Hkv, d, bs, lens, mb)
    got = oracle.decode_paged(q, kpool, vpool, table, lens, bs)
    for b, L in enumerate(lens):
        want = oracle.decode_cached(q[b:b + 1], kh[b][None], vh[b][None], L - n)
        assert np.array_equal(got[b:b + 1], want), b


def views_loop(q, kpool, vpool, table, lens, block_size):
    """The pages' loop order: per head and new token, walk the views by increasing Start,
    each clipped at the token's key limit startPos + qi + 1; scores are collected and
    normalized at the end (materialized softmax, float64)."""
    B, n, Hq, d = q.shape
    Hkv = kpool.shape[1]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, n, Hq, d))
    for b in range(B):
        L = lens[b]
        start = L - n
        nviews = -(-L // block_size)
        for h in range(Hq):
            g = h // G
            for qi in range(n):
                max_key = start + qi + 1
                scores, values = [], []
                for i in range(nviews):
                    v_start, v_len = i * block_size, min(block_size, L - i * block_size)
                    if v_start >= max_key:
                        continue
                    limit = min(v_len, max_key - v_start)
                    blk = table[b][i]
                    for t in range(limit):
                        scores.append(scale * sum(q[b, qi, h, e] * kpool[blk, g, t, e] for e in range(d)))
                        values.append(vpool[blk, g, t, :])
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                tot = sum(w)
                out[b, qi, h, :] = sum(wi * vi for wi, vi in zip(w, values)) / tot
    return out


@pytest.mark.parametrize("case", CASES[:3], ids=lambda c: "B%d-n%d-bs%d" % (c[0], c[1], c[5]))
def test_paged_matches_views_loop(case):
    B, n, Hq, Hkv, d, bs, lens, mb = case
    rng = np.random.default_rng(11)
    q, _, _, kpool, vpool, table = make_case(rng, B, n, Hq, Hkv, d, bs, lens, mb)
    got = oracle.decode_paged(q, kpool, vpool, table, lens, bs)
    want = views_loop(q, kpool, vpool, table, lens, bs)
    assert np.abs(got - want).max() <= 1e-12


def test_unused_table_entries_are_ignored():
    B, n, Hq, Hkv, d, bs, lens, mb = CASES[0]
    rng = np.random.default_rng(3)
    q, _, _, kpool, vpool, table = make_case(rng, B, n, Hq, Hkv, d, bs, lens, mb)
    base = oracle.decode_paged(q, kpool, vpool, table, lens, bs)
    t2 = table.copy()
    for b, L in enumerate(lens):
        t2[b, -(-L // bs):] = 10**6  # never a valid block
    assert np.array_equal(oracle.decode_paged(q, kpool, vpool, t2, lens, bs), base)


def test_shared_blocks_give_equal_rows():
    # two sequences whose tables name the same blocks, and the same queries
    rng = np.random.default_rng(5)
    bs, Hkv, d, Hq, n = 4, 2, 6, 4, 2
    kpool = rng.standard_normal((5, Hkv, bs, d))
    vpool = rng.standard_normal((5, Hkv, bs, d))
    table = np.array([[3, 0, 4], [3, 0, 4]])
    q1 = rng.standard_normal((1, n, Hq, d))
    q = np.concatenate([q1, q1])
    out = oracle.decode_paged(q, kpool, vpool, table, [11, 11], bs)
    assert np.array_equal(out[0], out[1])
    # a shorter sequence over a prefix of the same blocks sees only that prefix
    short = oracle.decode_paged(q1, kpool, vpool, table[:1], [6], bs)
    want = oracle.decode_cached(q1, np.concatenate([kpool[3], kpool[0]], axis=1)[None, :, :6],
                                np.concatenate([vpool[3], vpool[0]], axis=1)[None, :, :6], 4)
    assert np.array_equal(short, want)


def test_paged_oracle_rejects_bad_metadata():
    rng = np.random.default_rng(1)
    kpool = rng.standard_normal((3, 1, 4, 2))
    q = rng.standard_normal((1, 2, 1, 2))
    table = np.array([[0, 2]])
    with pytest.raises(ValueError):  # length below the number of new tokens
        oracle.decode_paged(q, kpool, kpool, table, [1], 4)
    with pytest.raises(ValueError):  # needs 3 blocks, the table has 2
        oracle.decode_paged(q, kpool, kpool, table, [9], 4)
    with pytest.raises(ValueError):  # a needed entry outside the pool
        oracle.decode_paged(q, kpool, kpool, np.array([[0, 3]]), [6], 4)
    with pytest.raises(ValueError):  # pool block size disagrees
        oracle.decode_paged(q, kpool, kpool, table, [6], 2)


# ---- planted mistakes in the gather must fail the pins ---------------------------------

def _bad_gather(kind):
    good = oracle.gather_paged

    def gather(pool, block_table, seq_len, block_size, b):
        pool = oracle.to_f64(pool)
        nblk = -(-seq_len // block_size)
        ids = [int(x) for x in np.asarray(block_table)[b, :nblk]]
        if kind == "reversed_blocks":
            ids = ids[::-1]
        if kind == "token_major_block":  # reads a block as [token][kvHead][d]
            blocks = [pool[i].reshape(block_size, pool.shape[1], -1).transpose(1, 0, 2) for i in ids]
            return np.concatenate(blocks, axis=1)[:, :seq_len]
        if kind == "drop_partial_block":
            nfull = seq_len // block_size
            hist = good(pool, block_table, seq_len, block_size, b)
            return hist if nfull * block_size == seq_len else hist[:, :nfull * block_size]
        if kind == "off_by_one_row":
            hist = np.concatenate([pool[i] for i in ids], axis=1)
            return hist[:, 1:seq_len + 1] if hist.shape[1] > seq_len else hist[:, :seq_len]
        return np.concatenate([pool[i] for i in ids], axis=1)[:, :seq_len]

    return gather


@pytest.mark.parametrize("kind", ["reversed_blocks", "token_major_block", "drop_partial_block",
                                  "off_by_one_row"])
def test_pins_catch_planted_gather_mistakes(monkeypatch, kind):
    B, n, Hq, Hkv, d, bs, lens, mb = CASES[1]
    rng = np.random.default_rng(7)
    q, kh, vh, kpool, vpool, table = make_case(rng, B, n, Hq, Hkv, d, bs, lens, mb)
    monkeypatch.setattr(oracle, "gather_paged", _bad_gather(kind))
    caught = 0
    try:
        got = oracle.decode_paged(q, kpool, vpool, table, lens, bs)
    except ValueError:
        got = None
    if got is None or np.isnan(got).any():
        caught += 1
    else:
        for b, L in enumerate(lens):
            want = oracle.decode_cached(q[b:b + 1], kh[b][None], vh[b][None], L - n)
            if not np.array_equal(got[b:b + 1], want):
                caught += 1
                break
        if np.abs(got - views_loop(q, kpool, vpool, table, lens, bs)).max() > 1e-12:
            caught += 1
    assert caught >= 1, kind
