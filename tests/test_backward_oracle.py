"""Pins of the row-statistics and backward oracle (oracle/backward.py), CPU only.

Riftco's "Two exact full-sequence algorithms": the memory-linear path saves one [B, H, T]
statistic per row and its backward recomputes the probabilities and applies the exact
softmax vector-Jacobian product; a context gradient yields query, key and value
gradients.  Each pin checks the oracle against something other than its own formulas:

* a library routine: PyTorch float64 autograd through scaled_dot_product_attention
  (with enable_gqa), causal and not;
* brute force: central finite differences of <dO, attention(Q, K, V)> through the
  forward C oracle, element by element on tiny inputs;
* closed forms and invariants: the worked example's row statistic log(2e + 1); key
  gradients of a row sum to zero (a shift shared by every key leaves the softmax
  unchanged); value gradients sum to the upstream gradients (rows of P sum to one);
  causality (key j's gradients ignore upstream rows before j; query i's ignore keys
  after i); GQA equals MHA with repeated K/V and head-summed K/V gradients.

Planted mistakes (no D term, a dropped scale, dK without the group sum, dV from the
unmasked scores, dK from dS instead of its transpose) must fail pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as bw


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def loss_grad_fd(q, k, v, dout, scale, causal, eps=1e-6):
    """Central differences of <dout, out> through the forward C oracle."""
    def L(q_, k_, v_):
        return float((oracle.prefill(q_, k_, v_, scale, causal) * dout).sum())
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            which = [a is x for a in (q, k, v)].index(True)
            args_p[which], args_m[which] = xp, xm
            g[idx] = (L(*args_p) - L(*args_m)) / (2 * eps)
        grads.append(g)
    return grads


def torch_grads(q, k, v, dout, scale, causal):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=scale,
                                                           enable_gqa=True)
    out.backward(torch.tensor(dout))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


# ---- pins, each a function of a backward implementation --------------------------------

def pin_torch_autograd(impl):
    ok = True
    for causal in (True, False):
        for (B, Hq, Hkv, T, d) in ((2, 4, 2, 9, 5), (1, 3, 1, 6, 4), (1, 2, 2, 5, 3)):
            q, k, v = rnd(1, B, Hq, T, d), rnd(2, B, Hkv, T, d), rnd(3, B, Hkv, T, d)
            do = rnd(4, B, Hq, T, d)
            got = impl(q, k, v, do, 0.7, causal)
            want = torch_grads(q, k, v, do, 0.7, causal)
            ok &= all(np.abs(a - b).max() < 1e-10 for a, b in zip(got, want))
    return ok


def pin_finite_differences(impl):
    B, Hq, Hkv, T, d = 1, 2, 1, 4, 3
    q, k, v = rnd(5, B, Hq, T, d), rnd(6, B, Hkv, T, d), rnd(7, B, Hkv, T, d)
    do = rnd(8, B, Hq, T, d)
    got = impl(q, k, v, do, 0.9, True)
    want = loss_grad_fd(q, k, v, do, 0.9, True)
    return all(np.abs(a - b).max() < 1e-6 for a, b in zip(got, want))


def pin_key_and_value_sums(impl):
    B, Hq, Hkv, T, d = 2, 6, 2, 11, 4
    q, k, v = rnd(9, B, Hq, T, d), rnd(10, B, Hkv, T, d), rnd(11, B, Hkv, T, d)
    do = rnd(12, B, Hq, T, d)
    dq, dk, dv = impl(q, k, v, do, 0.5, True)
    G = Hq // Hkv
    dk_sum_zero = np.abs(dk.sum(axis=2)).max() < 1e-10
    dv_sum = np.abs(dv.sum(axis=2) - do.reshape(B, Hkv, G, T, d).sum(axis=(2, 3))).max() < 1e-10
    return bool(dk_sum_zero and dv_sum)


def pin_causality(impl):
    B, Hq, Hkv, T, d = 1, 2, 1, 8, 3
    q, k, v = rnd(13, B, Hq, T, d), rnd(14, B, Hkv, T, d), rnd(15, B, Hkv, T, d)
    do = rnd(16, B, Hq, T, d)
    base = impl(q, k, v, do, 0.8, True)
    j = 5
    do2 = do.copy()
    do2[:, :, :j] += 3.0  # upstream rows before key j
    _, dk2, dv2 = impl(q, k, v, do2, 0.8, True)
    keys_ok = np.array_equal(dk2[:, :, j:], base[1][:, :, j:]) and np.array_equal(dv2[:, :, j:], base[2][:, :, j:])
    k3, v3 = k.copy(), v.copy()
    k3[:, :, j + 1:] += 2.0
    v3[:, :, j + 1:] -= 1.0
    dq3, _, _ = impl(q, k3, v3, do, 0.8, True)
    rows_ok = np.array_equal(dq3[:, :, :j + 1], base[0][:, :, :j + 1])
    return bool(keys_ok and rows_ok)


def pin_gqa_equals_mha(impl):
    B, Hq, Hkv, T, d = 1, 6, 2, 7, 4
    G = Hq // Hkv
    q, k, v = rnd(17, B, Hq, T, d), rnd(18, B, Hkv, T, d), rnd(19, B, Hkv, T, d)
    do = rnd(20, B, Hq, T, d)
    dq, dk, dv = impl(q, k, v, do, 0.6, True)
    dq_m, dk_m, dv_m = impl(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, 0.6, True)
    return bool(np.abs(dq - dq_m).max() < 1e-12
                and np.abs(dk - dk_m.reshape(B, Hkv, G, T, d).sum(axis=2)).max() < 1e-12
                and np.abs(dv - dv_m.reshape(B, Hkv, G, T, d).sum(axis=2)).max() < 1e-12)


PINS = [pin_torch_autograd, pin_finite_differences, pin_key_and_value_sums, pin_causality, pin_gqa_equals_mha]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_pins(pin):
    assert pin(bw.backward)


def test_lse_worked_example():
    """The primer's tiny example: q = (1, 0), keys (1,0), (0,1), (1,1), unscaled: scores
    1, 0, 1, so the row statistic is log(2e + 1) (its softmax denominator)."""
    k = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]).reshape(1, 1, 3, 2)
    qq = np.zeros((1, 1, 3, 2))
    qq[0, 0, 2] = [1.0, 0.0]
    got = bw.lse(qq, k, 1.0, True)
    assert abs(got[0, 0, 2] - math.log(2 * math.e + 1)) < 1e-14
    # row 0 sees key 0 only: lse = its score (q = 0 -> score 0)
    assert got[0, 0, 0] == 0.0


def test_lse_reconstructs_probabilities():
    """exp(s - lse) equals the oracle's probabilities, and rows sum to one."""
    q, k, v = rnd(21, 2, 4, 10, 6), rnd(22, 2, 2, 10, 6), rnd(23, 2, 2, 10, 6)
    L = bw.lse(q, k, 0.4, True)
    s = np.matmul(q, np.swapaxes(np.repeat(k, 2, axis=1), -1, -2)) * 0.4
    s = np.where(np.arange(10)[None, :] > np.arange(10)[:, None], -np.inf, s)
    P = np.exp(s - L[..., None])
    want = oracle.probs(q, k, v, 0.4, True)
    assert np.abs(P - want).max() < 1e-13
    assert np.abs(P.sum(-1) - 1).max() < 1e-13


# ---- planted mistakes ------------------------------------------------------------------

def _mutant(kind):
    def impl(q, k, v, dout, scale, causal=True):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        B, Hq, T, d = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        ke, ve = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
        P = bw.probs(q, k, scale, causal)
        Pv = bw.probs(q, k, scale, False) if kind == "dv_unmasked" else P
        dv_e = np.matmul(np.swapaxes(Pv, -1, -2), do)
        dP = np.matmul(do, np.swapaxes(ve, -1, -2))
        if kind == "no_d_term":
            dS = P * dP
        else:
            dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
        sc = 1.0 if kind == "dq_no_scale" else scale
        dq = sc * np.matmul(dS, ke)
        dk_e = scale * (np.matmul(dS, q) if kind == "dk_untransposed" else np.matmul(np.swapaxes(dS, -1, -2), q))
        if kind == "dk_first_head":
            dk = dk_e.reshape(B, Hkv, G, T, d)[:, :, 0]
        else:
            dk = dk_e.reshape(B, Hkv, G, T, d).sum(axis=2)
        dv = dv_e.reshape(B, Hkv, G, T, d).sum(axis=2)
        return dq, dk, dv
    return impl


@pytest.mark.parametrize("kind", ["no_d_term", "dq_no_scale", "dk_first_head", "dv_unmasked", "dk_untransposed"])
def test_backward_pins_catch_planted_mistakes(kind):
    failed = [p.__name__ for p in PINS if not p(_mutant(kind))]
    assert failed, kind
