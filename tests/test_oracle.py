"""Pins for the float64 oracle (CPU only).

Each pin checks the oracle against something other than itself: a value the
pages print, a closed form, an invariant the pages state, a library routine
(PyTorch's float64 scaled_dot_product_attention), or brute force.  The pins are
written as functions of an implementation so that the same pins can be shown
to catch planted mistakes (see test_pins_catch_planted_mistakes): a dropped
scale, a wrong GQA head map, an off-by-one causal mask, a softmax over the
wrong axis, a decode mask that ignores startPos.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ref_numpy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


class COracle:
    """The C oracle behind the pin interface."""

    @staticmethod
    def attention(q, k, v, scale, causal=True, pos0=0):
        return oracle.attention(q, k, v, scale, causal, pos0)

    @staticmethod
    def probs(q, k, v, scale, causal=True, pos0=0):
        return oracle.probs(q, k, v, scale, causal, pos0)


class NumpyOracle:
    @staticmethod
    def attention(q, k, v, scale, causal=True, pos0=0):
        return ref_numpy.attention(q, k, v, scale, causal, pos0)

    @staticmethod
    def probs(q, k, v, scale, causal=True, pos0=0):
        return ref_numpy.attention(q, k, v, scale, causal, pos0, return_probs=True)[1]


def rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- pins -----
# Each pin returns None when it holds and a short failure description otherwise.

def pin_worked_example(impl):
    """Multi-query attention primer, section 2.1 Tiny example: one query (1,0)
    over keys (1,0),(0,1),(1,1) with values 1,2,3, unscaled -> shares
    0.422/0.155/0.422 and output 2.0.  Closed form: output (4e+2)/(2e+1) = 2
    exactly; shares e/(2e+1) and 1/(2e+1)."""
    g = json.load(open(os.path.join(GOLDEN, "mqa_tiny_example.json")))
    K = np.array(g["K"])
    V = np.array(g["V"])
    # causal prefill, B=H=1, T=3, d=2: row 2 (position 2) sees all three keys.
    q = np.zeros((1, 1, 3, 2))
    q[0, 0, 2] = g["q"]
    q[0, 0, 0] = [0.3, -0.7]
    q[0, 0, 1] = [-1.1, 0.4]
    k = K.reshape(1, 1, 3, 2)
    v = np.zeros((1, 1, 3, 2))
    v[0, 0, :, 0] = V  # values padded to width 2 with zeros
    out = impl.attention(q, k, v, g["scale"], True, 0)
    P = impl.probs(q, k, v, g["scale"], True, 0)
    e = math.e
    want_w = np.array([e, 1.0, e]) / (2 * e + 1)
    if np.abs(P[0, 0, 2] - want_w).max() > 1e-15:
        return "shares %s != closed form %s" % (P[0, 0, 2], want_w)
    if [round(float(x), 3) for x in P[0, 0, 2]] != g["weights_rounded_3"]:
        return "shares do not round to the printed values"
    if abs(out[0, 0, 2, 0] - 2.0) > 1e-14 or out[0, 0, 2, 1] != 0.0:
        return "output %s != (2, 0)" % out[0, 0, 2]
    if round(float(out[0, 0, 2, 0]), 3) != g["output_rounded_3"]:
        return "output does not round to the printed value"
    # unmasked single-query form (causal off) gives the same
    out1 = impl.attention(np.array(g["q"]).reshape(1, 1, 1, 2), k, v, 1.0, False, 0)
    if abs(out1[0, 0, 0, 0] - 2.0) > 1e-14:
        return "non-causal single query output %s != 2" % out1[0, 0, 0, 0]
    # decode form: the query is the newest token at position 2, scale 1/sqrt(2),
    # so q = (sqrt 2, 0) reproduces the unscaled logits 1, 0, 1.
    qd = np.array([math.sqrt(2.0), 0.0]).reshape(1, 1, 1, 2)
    outd = impl.attention(qd, k, v, 1.0 / math.sqrt(2.0), True, 2)
    if abs(outd[0, 0, 0, 0] - 2.0) > 1e-14:
        return "decode output %s != 2" % outd[0, 0, 0, 0]
    return None


def pin_rows_sum_to_one_and_future_zero(impl):
    """Rows of P sum to one; every key after the query's position has
    probability exactly zero (Hesper "Causal Masking"; Riftco "The causal mask")."""
    rng = np.random.default_rng(1)
    for (B, Hq, Hkv, Tq, Tk, d, pos0) in [(2, 4, 2, 7, 7, 5, 0), (1, 3, 1, 3, 9, 4, 6), (1, 2, 2, 1, 5, 3, 4)]:
        q, k, v = rand(rng, B, Hq, Tq, d), rand(rng, B, Hkv, Tk, d), rand(rng, B, Hkv, Tk, d)
        P = impl.probs(q, k, v, 0.7, True, pos0)
        if np.abs(P.sum(-1) - 1.0).max() > 1e-12:
            return "rows do not sum to one"
        for i in range(Tq):
            fut = P[:, :, i, pos0 + i + 1:]
            if fut.size and np.any(fut != 0.0):
                return "non-zero probability on a future key (row %d)" % i
            if np.any(P[:, :, i, :pos0 + i + 1] <= 0.0):
                return "zero probability on an allowed key (row %d)" % i
    return None


def pin_causality(impl):
    """Outputs at position i do not change, bit for bit, when any q/k/v entry
    after position i changes (future tokens have no influence)."""
    rng = np.random.default_rng(2)
    B, Hq, Hkv, T, d = 2, 4, 2, 11, 6
    q, k, v = rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
    base = impl.attention(q, k, v, 0.4, True, 0)
    for t in (0, 3, 10):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, :, t + 1:] += 5.0 * rand(rng, B, Hq, T - t - 1, d)
        k2[:, :, t + 1:] -= 3.0
        v2[:, :, t + 1:] *= -7.0
        out = impl.attention(q2, k2, v2, 0.4, True, 0)
        if not np.array_equal(out[:, :, :t + 1], base[:, :, :t + 1]):
            return "rows <= %d changed when later tokens changed" % t
        if t + 1 < T and np.array_equal(out[:, :, t + 1:], base[:, :, t + 1:]):
            return "later rows did not change at all (perturbation ineffective)"
    return None


def pin_gqa_equals_mha(impl):
    """GQA with Hkv K/V heads equals MHA over K/V heads repeat-interleaved G
    times ("Grouped-Query Attention" 5.1: query heads 0 and 1 read the same
    K/V head).  Each K/V head has distinct data, so an h % Hkv map fails."""
    rng = np.random.default_rng(3)
    for (B, Hq, Hkv, T, d) in [(2, 6, 2, 8, 4), (1, 4, 1, 5, 3), (1, 8, 4, 6, 8)]:
        G = Hq // Hkv
        q, k, v = rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
        k += np.arange(Hkv).reshape(1, Hkv, 1, 1)
        a = impl.attention(q, k, v, 0.5, True, 0)
        ke = torch.from_numpy(k).repeat_interleave(G, dim=1).numpy()
        ve = torch.from_numpy(v).repeat_interleave(G, dim=1).numpy()
        b = impl.attention(q, ke, ve, 0.5, True, 0)
        if np.abs(a - b).max() > 1e-13:
            return "GQA != MHA with repeat_interleave for Hq=%d Hkv=%d" % (Hq, Hkv)
    return None


def pin_decode_equals_prefill_rows(impl):
    """Cached decode of n new tokens at startPos equals rows startPos..startPos+n-1
    of a full causal prefill over the same K/V (makarna's key limit
    startPos+qi+1 is the causal rule at absolute position startPos+qi)."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, T, d = 2, 4, 2, 13, 8
    q, k, v = rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
    s = 1 / math.sqrt(d)
    full = impl.attention(q, k, v, s, True, 0)
    for n in (1, 3, 13):
        sp = T - n
        dec = impl.attention(q[:, :, sp:], k, v, s, True, sp)
        if np.abs(dec - full[:, :, sp:]).max() > 1e-13:
            return "decode rows != prefill rows for n=%d" % n
    # a decode whose startPos is not at the end of the cache: keys beyond the
    # new tokens must be ignored
    dec = impl.attention(q[:, :, 5:7], k, v, s, True, 5)
    if np.abs(dec - full[:, :, 5:7]).max() > 1e-13:
        return "decode in the middle of the cache != prefill rows"
    return None


def pin_torch_sdpa(impl):
    """Library routine: PyTorch's float64 scaled_dot_product_attention (with
    enable_gqa for grouped heads) on random shapes, causal and not."""
    rng = np.random.default_rng(5)
    F = torch.nn.functional
    for (B, Hq, Hkv, T, d, causal, scale) in [(2, 4, 2, 9, 5, True, 0.3), (1, 6, 3, 17, 8, True, 1 / math.sqrt(8)),
                                              (2, 3, 1, 6, 3, False, 0.9), (1, 2, 2, 33, 16, True, 0.25)]:
        q, k, v = rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
        want = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                              is_causal=causal, scale=scale, enable_gqa=True).numpy()
        got = impl.attention(q, k, v, scale, causal, 0)
        if np.abs(got - want).max() > 1e-12:
            return "differs from torch SDPA (B%d Hq%d Hkv%d T%d d%d causal=%s): %g" % (
                B, Hq, Hkv, T, d, causal, np.abs(got - want).max())
    return None


def pin_closed_forms(impl):
    """scale 0 gives uniform weights: causal output at row i is the mean of
    v[0..i] (non-causal: the mean of all rows); T=1 returns v[0] exactly."""
    rng = np.random.default_rng(6)
    B, Hq, Hkv, T, d = 1, 4, 2, 10, 3
    q, k, v = rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
    out = impl.attention(q, k, v, 0.0, True, 0)
    ve = np.repeat(v, 2, axis=1)
    prefix = np.cumsum(ve, axis=2) / np.arange(1, T + 1).reshape(1, 1, T, 1)
    if np.abs(out - prefix).max() > 1e-14:
        return "scale=0 causal output is not the prefix mean"
    out = impl.attention(q, k, v, 0.0, False, 0)
    if np.abs(out - ve.mean(axis=2, keepdims=True)).max() > 1e-14:
        return "scale=0 non-causal output is not the column mean"
    out = impl.attention(q[:, :, :1], k[:, :, :1], v[:, :, :1], 0.8, True, 0)
    if not np.array_equal(out, np.repeat(v[:, :, :1], 2, axis=1)):
        return "T=1 output is not v[0]"
    return None


def pin_large_logits_and_shift(impl):
    """Peaky rows (q scaled by 64) stay finite and agree with torch's float64
    SDPA; adding the same constant to every score of a row (through a shared
    extra key component) leaves the output unchanged."""
    rng = np.random.default_rng(7)
    F = torch.nn.functional
    B, Hq, Hkv, T, d = 1, 2, 1, 12, 4
    q, k, v = rand(rng, B, Hq, T, d) * 64, rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
    got = impl.attention(q, k, v, 0.5, True, 0)
    if not np.all(np.isfinite(got)):
        return "non-finite output for large logits"
    want = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                          is_causal=True, scale=0.5, enable_gqa=True).numpy()
    if np.abs(got - want).max() > 1e-10:
        return "large-logit output differs from torch SDPA"
    q2 = np.concatenate([q / 64, np.full((B, Hq, T, 1), 3.0)], axis=-1)
    k2 = np.concatenate([k, np.full((B, Hkv, T, 1), 25.0)], axis=-1)  # +37.5 on every score
    a = impl.attention(q2[..., :d], k, v, 0.5, True, 0)
    b = impl.attention(q2, k2, np.concatenate([v, np.zeros((B, Hkv, T, 1))], -1), 0.5, True, 0)[..., :d]
    if np.abs(a - b).max() > 1e-12:
        return "shifting every score of a row changed the output"
    return None


PINS = [pin_worked_example, pin_rows_sum_to_one_and_future_zero, pin_causality, pin_gqa_equals_mha,
        pin_decode_equals_prefill_rows, pin_torch_sdpa, pin_closed_forms, pin_large_logits_and_shift]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_c_oracle_pins(pin):
    assert pin(COracle) is None


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_numpy_oracle_pins(pin):
    assert pin(NumpyOracle) is None


def test_c_oracle_brute_force_vs_numpy():
    """The two oracles agree on a grid of tiny shapes, with N(0,1) and
    integer-valued inputs (B<=2, Hkv in {1,2}, G in {1,2,3}, T<=9, d in {1,2,3,8})."""
    rng = np.random.default_rng(8)
    worst = 0.0
    for B in (1, 2):
        for Hkv in (1, 2):
            for G in (1, 2, 3):
                for T in (1, 2, 5, 9):
                    for d in (1, 2, 3, 8):
                        for causal in (True, False):
                            Hq = Hkv * G
                            if rng.random() < 0.5:
                                q, k, v = (rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d),
                                           rand(rng, B, Hkv, T, d))
                            else:
                                q = rng.integers(-3, 4, (B, Hq, T, d)).astype(float)
                                k = rng.integers(-3, 4, (B, Hkv, T, d)).astype(float)
                                v = rng.integers(-3, 4, (B, Hkv, T, d)).astype(float)
                            s = 1 / math.sqrt(d)
                            a = oracle.attention(q, k, v, s, causal, 0)
                            b = ref_numpy.attention(q, k, v, s, causal, 0)
                            worst = max(worst, float(np.abs(a - b).max()))
    assert worst <= 1e-12, worst


def test_oracle_rejects_bad_arguments():
    q = np.zeros((1, 3, 4, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, 1.0)  # Hq % Hkv != 0
    q = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, 1.0, True, 1)  # startPos + newTokens > totalLen


def test_oracle_threads_do_not_change_result():
    rng = np.random.default_rng(9)
    q, k, v = rand(rng, 2, 8, 33, 16), rand(rng, 2, 4, 33, 16), rand(rng, 2, 4, 33, 16)
    a = oracle.attention(q, k, v, 0.25, True, 0, nthreads=1)
    b = oracle.attention(q, k, v, 0.25, True, 0, nthreads=5)
    assert np.array_equal(a, b)


def test_decode_wrapper_layout():
    """decode_cached takes q/out token-major [B,n,Hq,d] and caches head-major."""
    rng = np.random.default_rng(10)
    B, n, Hq, Hkv, L, d = 2, 3, 4, 2, 9, 8
    qt = rand(rng, B, n, Hq, d)
    kc, vc = rand(rng, B, Hkv, L, d), rand(rng, B, Hkv, L, d)
    out = oracle.decode_cached(qt, kc, vc, L - n)
    ref = ref_numpy.attention(qt.transpose(0, 2, 1, 3), kc, vc, 1 / math.sqrt(d), True, L - n)
    assert np.abs(out - ref.transpose(0, 2, 1, 3)).max() < 1e-13


# ------------------------------------------- algorithm checks (CPU, float64) --
# The GPU kernels do not materialize the score row: they run the online
# softmax recurrence over key tiles and, in decode, split the keys into chunks
# whose partial (max, sum, numerator) triples are merged with log-sum-exp
# algebra.  Both are exact in exact arithmetic; these float64 loops show it
# against the oracle before any GPU code is trusted.

def online_softmax_attention(q, k, v, scale, causal, pos0, tile):
    """Online recurrence over key tiles (running max m, normalizer l, numerator o)."""
    B, Hq, Tq, d = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Tq):
                m, l, o = -np.inf, 0.0, np.zeros(d)
                lim = min(Tk, pos0 + i + 1) if causal else Tk
                for j0 in range(0, lim, tile):
                    j1 = min(lim, j0 + tile)
                    s = k[b, g, j0:j1] @ q[b, h, i] * scale
                    m_new = max(m, s.max())
                    alpha = math.exp(m - m_new) if m > -np.inf else 0.0
                    p = np.exp(s - m_new)
                    l = alpha * l + p.sum()
                    o = alpha * o + p @ v[b, g, j0:j1]
                    m = m_new
                out[b, h, i] = o / l
    return out


def split_kv_attention(q, k, v, scale, pos0, bounds):
    """Split the key axis at `bounds`, compute a partial (m, l, o) per chunk,
    then merge: M = max m_s, L = sum l_s e^(m_s-M), O = sum o_s e^(m_s-M) / L."""
    B, Hq, Tq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Tq):
                lim = pos0 + i + 1
                parts = []
                for c0, c1 in zip(bounds[:-1], bounds[1:]):
                    c1 = min(c1, lim)
                    if c1 <= c0:
                        continue
                    s = k[b, g, c0:c1] @ q[b, h, i] * scale
                    m = s.max()
                    p = np.exp(s - m)
                    parts.append((m, p.sum(), p @ v[b, g, c0:c1]))
                M = max(p[0] for p in parts)
                L = sum(l * math.exp(m - M) for m, l, _ in parts)
                O = sum(o * math.exp(m - M) for m, _, o in parts)
                out[b, h, i] = O / L
    return out


def test_online_recurrence_matches_oracle():
    rng = np.random.default_rng(11)
    q, k, v = rand(rng, 1, 4, 21, 8), rand(rng, 1, 2, 21, 8), rand(rng, 1, 2, 21, 8)
    want = oracle.attention(q, k, v, 0.35, True, 0)
    for tile in (1, 4, 16, 64):
        assert np.abs(online_softmax_attention(q, k, v, 0.35, True, 0, tile) - want).max() < 1e-12


def test_split_kv_merge_matches_oracle():
    rng = np.random.default_rng(12)
    L, n = 40, 4
    q, k, v = rand(rng, 2, 4, n, 8) * 3, rand(rng, 2, 1, L, 8), rand(rng, 2, 1, L, 8)
    want = oracle.attention(q, k, v, 0.35, True, L - n)
    for _ in range(5):
        cuts = sorted(set(rng.integers(1, L, 4).tolist()))
        bounds = [0] + cuts + [L]
        got = split_kv_attention(q, k, v, 0.35, L - n, bounds)
        assert np.abs(got - want).max() < 1e-12


# ------------------------------------------------------ planted mistakes --
# Mutants of the NumPy oracle, each carrying one plausible mistake.  Every
# mutant must fail at least one pin, which shows the pins above can see it.

def _mutant(kind):
    def attention(q, k, v, scale, causal=True, pos0=0, return_probs=False):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, Tq, d = q.shape
        Hkv, Tk = k.shape[1], k.shape[2]
        G = Hq // Hkv
        if kind == "head_mod":
            idx = np.arange(Hq) % Hkv
        else:
            idx = np.arange(Hq) // G
        ke, ve = k[:, idx], v[:, idx]
        if kind == "v_head_mod":
            ve = v[:, np.arange(Hq) % Hkv]
        sc = 1.0 if kind == "no_scale" else scale
        s = np.matmul(q, np.swapaxes(ke, -1, -2)) * sc
        if causal:
            p0 = 0 if kind == "ignore_pos0" else pos0
            pos = p0 + np.arange(Tq)[:, None]
            keys = np.arange(Tk)[None, :]
            masked = keys >= pos if kind == "strict_mask" else keys > pos
            s = np.where(masked, -np.inf, s)
        axis = -2 if kind == "wrong_axis" else -1
        s = s - s.max(axis=axis, keepdims=True)
        w = np.exp(s)
        p = w / w.sum(axis=axis, keepdims=True)
        p = np.nan_to_num(p)
        out = np.matmul(p, ve)
        return (out, p) if return_probs else out

    class M:
        @staticmethod
        def attention(q, k, v, scale, causal=True, pos0=0):
            return attention(q, k, v, scale, causal, pos0)

        @staticmethod
        def probs(q, k, v, scale, causal=True, pos0=0):
            return attention(q, k, v, scale, causal, pos0, True)[1]

    return M


@pytest.mark.parametrize("kind", ["head_mod", "v_head_mod", "no_scale", "strict_mask", "wrong_axis",
                                  "ignore_pos0"])
def test_pins_catch_planted_mistakes(kind):
    impl = _mutant(kind)
    failures = []
    for pin in PINS:
        try:
            r = pin(impl)
        except Exception as e:  # a crash also counts as a caught mistake
            r = "raised %r" % e
        if r is not None:
            failures.append(pin.__name__)
    assert failures, "planted mistake %r passed every pin" % kind


def test_c_oracle_never_reads_masked_values():
    """Future value rows are not part of row i's sum at all (not even as 0 * v):
    a NaN planted after position t leaves every row before t finite."""
    rng = np.random.default_rng(13)
    q, k, v = rand(rng, 1, 2, 9, 4), rand(rng, 1, 1, 9, 4), rand(rng, 1, 1, 9, 4)
    v[0, 0, 5, 1] = np.nan
    k[0, 0, 6, 2] = np.nan
    o = oracle.attention(q, k, v, 0.5, True, 0)
    assert np.isfinite(o[0, :, :5]).all()
    assert np.isnan(o[0, :, 5:]).any(-1).all()
