"""Pins of local (sliding-window) causal attention in both float64 oracles, on the CPU.

Local attention restricts each query to its own position and the window-1 before it
(the multi-query primer, section 4.1: decoder self-attention limited to the current
position and the previous 31 positions, i.e. window 32).  Each pin checks the oracles
against something other than themselves: a slice of the keys attended without any
mask, the exact W = 1 and W >= T special cases, the closed form at scale 0, the
support of P, a brute-force grid between the two oracles, and the decode / paged
wrappers against the prefill rows.  Planted window mistakes must fail the pins.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ref_numpy


def c_impl(q, k, v, scale, causal=True, pos0=0, window=0):
    return oracle.attention(q, k, v, scale, causal, pos0, window=window)


def np_impl(q, k, v, scale, causal=True, pos0=0, window=0):
    return ref_numpy.attention(q, k, v, scale, causal, pos0, window=window)


def rand(rng, *shape):
    return rng.standard_normal(shape)


def pin_slice(impl):
    """Row i of a window-W attention = unmasked attention of q_i over keys i-W+1..i."""
    rng = np.random.default_rng(1)
    B, Hq, Hkv, T, d = 2, 4, 2, 23, 5
    q, k, v = rand(rng, B, Hq, T, d), rand(rng, B, Hkv, T, d), rand(rng, B, Hkv, T, d)
    for W in (1, 3, 8, 22):
        got = impl(q, k, v, 0.7, True, 0, W)
        for i in (0, 1, W - 1, W, T - 1):
            if i >= T:
                continue
            lo = max(0, i - W + 1)
            want = oracle.attention(q[:, :, i:i + 1], k[:, :, lo:i + 1], v[:, :, lo:i + 1], 0.7, False)
            if np.abs(got[:, :, i] - want[:, :, 0]).max() > 1e-12:
                return False
    return True


def pin_window_one_is_own_value(impl):
    rng = np.random.default_rng(2)
    q, k, v = rand(rng, 1, 2, 9, 4), rand(rng, 1, 1, 9, 4), rand(rng, 1, 1, 9, 4)
    got = impl(q, k, v, 1.3, True, 0, 1)
    return bool(np.array_equal(got, np.repeat(v, 2, axis=1)))


def pin_wide_window_is_causal(impl):
    rng = np.random.default_rng(3)
    q, k, v = rand(rng, 1, 2, 12, 4), rand(rng, 1, 2, 12, 4), rand(rng, 1, 2, 12, 4)
    full = impl(q, k, v, 0.5, True, 0, 0)
    return all(np.array_equal(impl(q, k, v, 0.5, True, 0, W), full) for W in (12, 13, 1000))


def pin_scale_zero_window_mean(impl):
    rng = np.random.default_rng(4)
    T, W = 15, 4
    q, k, v = rand(rng, 1, 1, T, 3), rand(rng, 1, 1, T, 3), rand(rng, 1, 1, T, 3)
    got = impl(q, k, v, 0.0, True, 0, W)
    want = np.stack([v[0, 0, max(0, i - W + 1):i + 1].mean(axis=0) for i in range(T)])
    return np.abs(got[0, 0] - want).max() <= 1e-14


def pin_decode_rows(impl):
    """Rows at pos0 = startPos.. of a window decode = the same rows of window prefill."""
    rng = np.random.default_rng(5)
    T, n, W = 20, 3, 6
    q, k, v = rand(rng, 1, 4, T, 4), rand(rng, 1, 2, T, 4), rand(rng, 1, 2, T, 4)
    full = impl(q, k, v, 0.4, True, 0, W)
    dec = impl(q[:, :, T - n - 4:T - 4], k, v, 0.4, True, T - n - 4, W)
    return np.abs(dec - full[:, :, T - n - 4:T - 4]).max() <= 1e-12


PINS = [pin_slice, pin_window_one_is_own_value, pin_wide_window_is_causal,
        pin_scale_zero_window_mean, pin_decode_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
@pytest.mark.parametrize("impl", [c_impl, np_impl], ids=["c", "numpy"])
def test_window_pins(impl, pin):
    assert pin(impl)


def test_primer_window_32_support():
    """Window 32 (the primer's local decoder): P row i is nonzero exactly on keys
    max(0, i-31) .. i."""
    rng = np.random.default_rng(6)
    T = 70
    q, k, v = rand(rng, 1, 1, T, 4), rand(rng, 1, 1, T, 4), rand(rng, 1, 1, T, 4)
    P = oracle.probs(q, k, v, 0.5, True, 0, window=32)[0, 0]
    for i in range(T):
        nz = np.nonzero(P[i])[0]
        assert nz[0] == max(0, i - 31) and nz[-1] == i and len(nz) == min(i + 1, 32)
        assert abs(P[i].sum() - 1) <= 1e-12


def test_c_vs_numpy_brute_force_window():
    rng = np.random.default_rng(7)
    worst = 0.0
    for B in (1, 2):
        for Hkv in (1, 2):
            for G in (1, 3):
                for T in (1, 5, 9):
                    for W in (1, 2, 4, 9):
                        q = rand(rng, B, Hkv * G, T, 3)
                        k, v = rand(rng, B, Hkv, T, 3), rand(rng, B, Hkv, T, 3)
                        a = c_impl(q, k, v, 0.8, True, 0, W)
                        b = np_impl(q, k, v, 0.8, True, 0, W)
                        worst = max(worst, float(np.abs(a - b).max()))
    assert worst <= 1e-12


def test_window_through_decode_and_paged_wrappers():
    rng = np.random.default_rng(8)
    B, n, Hq, Hkv, d, L, W = 2, 3, 4, 2, 6, 40, 7
    q = rand(rng, B, n, Hq, d)
    kc, vc = rand(rng, B, Hkv, L, d), rand(rng, B, Hkv, L, d)
    dec = oracle.decode_cached(q, kc, vc, L - n, window=W)
    pre = oracle.attention(q.transpose(0, 2, 1, 3), kc, vc, 1 / math.sqrt(d), True, L - n, window=W)
    assert np.array_equal(dec, pre.transpose(0, 2, 1, 3))
    bs = 8
    table = np.array([[4, 0, 2, 1, 3], [9, 5, 8, 6, 7]])
    kp = np.full((10, Hkv, bs, d), np.nan)
    vp = np.full((10, Hkv, bs, d), np.nan)
    for b in range(B):
        for p_ in range(L):
            kp[table[b, p_ // bs], :, p_ % bs] = kc[b, :, p_]
            vp[table[b, p_ // bs], :, p_ % bs] = vc[b, :, p_]
    pag = oracle.decode_paged(q, kp, vp, table, [L, L], bs, window=W)
    assert np.array_equal(pag, dec)


def test_window_rejections():
    rng = np.random.default_rng(9)
    q, k = rand(rng, 1, 1, 4, 2), rand(rng, 1, 1, 4, 2)
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, 1.0, False, 0, window=2)  # window needs causal
    with pytest.raises(ValueError):
        oracle.attention(q, k, k, 1.0, True, 0, window=-1)
    with pytest.raises(ValueError):
        ref_numpy.attention(q, k, k, 1.0, False, 0, window=2)


# ---- planted window mistakes -------------------------------------------------------------

def _mutant(kind):
    def impl(q, k, v, scale, causal=True, pos0=0, window=0):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, Hq, Tq, d = q.shape
        G = Hq // k.shape[1]
        ke, ve = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        s = np.matmul(q, np.swapaxes(ke, -1, -2)) * scale
        pos = pos0 + np.arange(Tq)[:, None]
        keys = np.arange(k.shape[2])[None, :]
        bias = np.where(keys > pos, -np.inf, 0.0)
        if window:
            if kind == "window_too_wide":
                lo = pos - window
            elif kind == "window_too_narrow":
                lo = pos - window + 2
            elif kind == "window_from_zero":
                lo = np.zeros_like(pos) + (Tq - window if Tq > window else 0)
            else:  # "window_ignores_pos0"
                lo = np.arange(Tq)[:, None] - window + 1
            bias = np.where(keys < lo, -np.inf, bias)
        s = s + bias
        s = s - s.max(axis=-1, keepdims=True)
        w = np.exp(s)
        return np.matmul(w / w.sum(axis=-1, keepdims=True), ve)
    return impl


@pytest.mark.parametrize("kind", ["window_too_wide", "window_too_narrow", "window_from_zero",
                                  "window_ignores_pos0"])
def test_window_pins_catch_planted_mistakes(kind):
    impl = _mutant(kind)
    failed = [p.__name__ for p in PINS if not p(impl)]
    assert failed, kind
