"""Pins of the KV-cache append oracle (NeoX RoPE on K + cache write), CPU only.

The pages describe the fused step (Hesper's fused RoPE-K + KV cache write: the rotation
pair of dim j is dim j + d/2, the angle grows with the absolute position and falls with
the pair index; forge's apply_rope with offset = start_pos before the cache append) but
do not render its equations.  Each pin checks the oracle against something other than
its own formula:

* a library routine: the rotate-half rotary embedding of the transformers package
  (its rotary-frequency schedule at small positions, and its pairing applied to the
  oracle's own cos/sin);
* invariants of a rotary embedding: the norm of every rotation pair is kept, position 0
  is the identity, and the score between a rotated query and key depends only on their
  distance (shifting both positions changes nothing);
* the per-pair frequency factor acts as a position divisor for its pair alone;
* the cache write: rows outside the new positions are untouched, V rows are copied,
  and the paged write agrees with the contiguous one position by position.

Planted mistakes in the rotation (interleaved pairs, a flipped sign, the wrong
frequency exponent, a multiplied frequency factor, an off-by-one position) must fail
at least one pin.
"""
import numpy as np
import pytest
import torch

from oracle import kv_append as ka


def rng(seed):
    return np.random.default_rng(seed)


# ---- the rotation ------------------------------------------------------------------

def pin_library_frequencies(rope):
    """transformers' rotary embedding (rope_theta = base) at positions 0..63."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    d, base = 64, 10000.0
    cfg = LlamaConfig(hidden_size=d * 2, num_attention_heads=2, head_dim=d, rope_theta=base,
                      max_position_embeddings=256)
    emb = LlamaRotaryEmbedding(cfg)
    pos = np.arange(64)
    x = rng(1).standard_normal((1, 1, 64, d))
    xt = torch.from_numpy(x).to(torch.float32)
    cos, sin = emb(xt, torch.from_numpy(pos)[None])
    want, _ = apply_rotary_pos_emb(xt, xt, cos, sin)
    got = rope(x, pos, base)
    return float(np.abs(got - want.double().numpy()).max()) < 2e-4


def pin_library_pairing(rope):
    """The rotate-half pairing of transformers, in float64 with exact cos/sin."""
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb

    d, base = 16, 500.0
    pos = np.array([0, 1, 5, 77, 1000, 32767])
    x = rng(2).standard_normal((2, 3, len(pos), d))
    ang = ka.rope_angles(pos, d, base)
    emb = np.concatenate([ang, ang], axis=-1)  # the library's [T, d] angle layout
    cos = torch.from_numpy(np.cos(emb))[None]
    sin = torch.from_numpy(np.sin(emb))[None]
    xt = torch.from_numpy(x)
    want, _ = apply_rotary_pos_emb(xt, xt, cos, sin, unsqueeze_dim=1)
    return float(np.abs(rope(x, pos, base) - want.numpy()).max()) < 1e-12


def pin_pair_norms_and_identity(rope):
    d = 12
    x = rng(3).standard_normal((4, 9, d))
    pos = np.arange(9) * 37
    y = rope(x, pos, 10000.0)
    h = d // 2
    n_x = x[..., :h] ** 2 + x[..., h:] ** 2
    n_y = y[..., :h] ** 2 + y[..., h:] ** 2
    ident = rope(x[:, :1], np.zeros(1), 10000.0)
    return bool(np.abs(n_x - n_y).max() < 1e-12 and np.array_equal(ident, x[:, :1]))


def pin_relative_position(rope):
    """<R(q, m), R(k, n)> depends on m - n only."""
    d = 32
    q = rng(4).standard_normal(d)
    k = rng(5).standard_normal(d)
    def score(m, n):
        return float(rope(q[None], np.array([m]), 10000.0)[0] @ rope(k[None], np.array([n]), 10000.0)[0])
    ok = True
    for m, n in ((5, 2), (100, 99), (3, 40)):
        for shift in (1, 17, 4096):
            ok &= abs(score(m, n) - score(m + shift, n + shift)) < 1e-9
    # and it does depend on the distance
    ok &= abs(score(5, 2) - score(5, 3)) > 1e-6
    return ok


def pin_distinct_pair_frequencies(rope):
    """At position 1 pair j turns by a distinct, decreasing angle: unit vectors e_j."""
    d, base = 16, 10000.0
    h = d // 2
    eye = np.eye(d)[:h]  # e_j for j < d/2 rotates inside pair j
    y = rope(eye[:, None, :], np.array([1]), base)[:, 0, :]
    ang = np.arctan2(y[np.arange(h), np.arange(h) + h], y[np.arange(h), np.arange(h)])
    # pair 0 turns by exactly one radian per position; the angles fall geometrically
    ratio = ang[1:] / ang[:-1]
    return bool(abs(ang[0] - 1.0) < 1e-12 and np.all(np.abs(ratio - ratio[0]) < 1e-9)
                and abs(ratio[0] - base ** (-2.0 / d)) < 1e-9)


def pin_freq_factor_divides_position(rope):
    d, base = 8, 10000.0
    ff = np.array([1.0, 2.0, 4.0, 8.0])
    x = rng(6).standard_normal((1, 1, d))
    got = rope(x, np.array([40]), base, ff)
    ok = True
    for j, f in enumerate(ff):
        want = rope(x, np.array([40.0 / f]), base)
        ok &= abs(got[0, 0, j] - want[0, 0, j]) < 1e-12 and abs(got[0, 0, j + 4] - want[0, 0, j + 4]) < 1e-12
    return ok


PINS = [pin_library_frequencies, pin_library_pairing, pin_pair_norms_and_identity,
        pin_relative_position, pin_distinct_pair_frequencies, pin_freq_factor_divides_position]


def oracle_rope(x, pos, base, ff=None):
    return ka.rope_neox(x, pos, base, ff)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_rope_pins(pin):
    assert pin(oracle_rope)


def _mutant(kind):
    def rope(x, pos, base, ff=None):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        h = d // 2
        j = np.arange(h)
        expo = -1.0 * j / d if kind == "exponent" else -2.0 * j / d
        inv = np.power(base, expo)
        if ff is not None:
            inv = inv * ff if kind == "factor_multiplies" else inv / ff
        p = np.asarray(pos, dtype=np.float64) + (1 if kind == "position_off_by_one" else 0)
        a = p[:, None] * inv[None, :]
        c, s = np.cos(a), np.sin(a)
        if kind == "interleaved":
            x1, x2 = x[..., 0::2], x[..., 1::2]
            y = np.empty_like(x)
            y[..., 0::2] = x1 * c - x2 * s
            y[..., 1::2] = x2 * c + x1 * s
            return y
        x1, x2 = x[..., :h], x[..., h:]
        if kind == "sign":
            return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], axis=-1)
        return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
    return rope


@pytest.mark.parametrize("kind", ["interleaved", "sign", "exponent", "factor_multiplies",
                                  "position_off_by_one"])
def test_rope_pins_catch_planted_mistakes(kind):
    failed = [p.__name__ for p in PINS if not p(_mutant(kind))]
    assert failed, kind


# ---- the cache write ---------------------------------------------------------------

def test_append_rows_and_untouched_rows():
    r = rng(7)
    B, Hkv, L, d, n, sp = 2, 3, 20, 8, 4, 9
    kc, vc = r.standard_normal((B, Hkv, L, d)), r.standard_normal((B, Hkv, L, d))
    kn, vn = r.standard_normal((B, n, Hkv, d)), r.standard_normal((B, n, Hkv, d))
    k2, v2 = ka.kv_append(kc, vc, kn, vn, sp, rope_base=10000.0)
    keep = np.r_[0:sp, sp + n:L]
    assert np.array_equal(k2[:, :, keep], kc[:, :, keep]) and np.array_equal(v2[:, :, keep], vc[:, :, keep])
    assert np.array_equal(v2[:, :, sp:sp + n], np.swapaxes(vn, 1, 2))
    # row sp+i of head g is token i's K of head g rotated at position sp+i
    for b in range(B):
        for g in range(Hkv):
            for i in range(n):
                want = ka.rope_neox(kn[b, i, g][None], np.array([sp + i]), 10000.0)[0]
                assert np.abs(k2[b, g, sp + i] - want).max() < 1e-12
    # no RoPE: plain copy
    k3, _ = ka.kv_append(kc, vc, kn, vn, sp, rope_base=0.0)
    assert np.array_equal(k3[:, :, sp:sp + n], np.swapaxes(kn, 1, 2))
    # inputs untouched
    assert not np.shares_memory(k2, kc)


def test_append_rejects_overflow():
    z = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        ka.kv_append(z, z, np.zeros((1, 2, 1, 2)), np.zeros((1, 2, 1, 2)), 3)
    with pytest.raises(ValueError):
        ka.rope_angles(np.arange(2), 3, 10000.0)


def test_paged_append_matches_contiguous():
    r = rng(8)
    B, Hkv, d, n, bs = 3, 2, 8, 3, 4
    lens = [3, 9, 16]
    maxb = 4
    nblk = 14
    perm = r.permutation(nblk)
    table = -np.ones((B, maxb), dtype=np.int64)
    c = 0
    for b in range(B):
        for i in range((lens[b] + bs - 1) // bs):
            table[b, i] = perm[c]
            c += 1
    kp, vp = r.standard_normal((nblk, Hkv, bs, d)), r.standard_normal((nblk, Hkv, bs, d))
    kn, vn = r.standard_normal((B, n, Hkv, d)), r.standard_normal((B, n, Hkv, d))
    ff = np.linspace(1.0, 3.0, d // 2)
    k2, v2 = ka.kv_append_paged(kp, vp, table, lens, kn, vn, 500.0, ff)
    for b in range(B):
        L = lens[b]
        # the contiguous view of this sequence before and after
        kc = np.stack([kp[table[b, p // bs], :, p % bs] for p in range(L)], axis=1)[None]
        vc = np.stack([vp[table[b, p // bs], :, p % bs] for p in range(L)], axis=1)[None]
        kw, vw = ka.kv_append(kc, vc, kn[b:b + 1], vn[b:b + 1], L - n, 500.0, ff)
        for p in range(L):
            assert np.array_equal(k2[table[b, p // bs], :, p % bs], kw[0, :, p])
            assert np.array_equal(v2[table[b, p // bs], :, p % bs], vw[0, :, p])
    # blocks no sequence owns keep their values
    owned = set(table[table >= 0].tolist())
    for blk in range(nblk):
        if blk not in owned:
            assert np.array_equal(k2[blk], kp[blk]) and np.array_equal(v2[blk], vp[blk])
