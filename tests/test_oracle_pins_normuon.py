"""Pins of the oracle's NorMuon scaling and cautious weight decay (the
web3.cnoyu.systems review of karpathy/autoresearch's train.py, the paragraph
after the Muon one) against facts that do not come from the
oracle itself: closed forms on orthonormal rows and columns, the RMS
normalisation that beta2 = 0 implies, the two-step moving average, transpose
equivariance, a hand-derived decay example and the special cases of the
mask.  Planted mistakes (wrong axis, sum for mean, missing square root, a
strict mask, decay after the update) each fail one of them."""
import math

import numpy as np
import pytest

import oracle
from oracle import muon_oracle as mo
import workloads as wl

QUINTIC = [wl.QUINTIC] * 5


def rng(seed):
    return np.random.default_rng(seed)


def orthonormal_rows(m, n, seed):
    """m x n (m <= n) with orthonormal rows: each row has unit norm by
    construction (QR), so its mean square along the row is 1/n exactly."""
    q, _ = np.linalg.qr(rng(seed).standard_normal((n, m)))
    return q.T


# ------------------------------------------------------------------ NorMuon
@pytest.mark.parametrize("m,n", [(4, 16), (8, 8), (1, 5), (32, 96)])
def test_normuon_closed_form_on_orthonormal_rows(m, n):
    q = orthonormal_rows(m, n, m * 100 + n)
    v0 = rng(1).uniform(0.0, 0.1, size=m)
    beta2, eps = 0.9, 1e-8
    o, v = mo.normuon_scale(q, v0, beta2, eps)
    v_expect = beta2 * v0 + (1 - beta2) / n
    assert np.allclose(v, v_expect, rtol=1e-13, atol=0)
    assert np.allclose(o * (np.sqrt(v_expect) + eps)[:, None], q, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("n,m", [(16, 4), (5, 1), (96, 32)])
def test_normuon_tall_uses_columns(n, m):
    # a tall matrix with orthonormal columns: the statistics are per column
    q = orthonormal_rows(m, n, n * 7 + m).T
    v0 = np.zeros(m)
    o, v = mo.normuon_scale(q, v0, 0.5, 0.0)
    assert np.allclose(v, 0.5 / n, rtol=1e-13)
    assert np.allclose(o, q / math.sqrt(0.5 / n), rtol=1e-12)


@pytest.mark.parametrize("shape", [(3, 7), (7, 3), (6, 6), (1, 9), (9, 1)])
def test_normuon_beta2_zero_normalises_rms(shape):
    # beta2 = 0, eps = 0: O' = O / rms along the longer side, so every
    # short-side slice of O' has mean square 1
    o = rng(sum(shape)).standard_normal(shape)
    o2, v = mo.normuon_scale(o, np.full(min(shape), 123.0), 0.0, 0.0)
    axis = 0 if shape[0] > shape[1] else 1
    assert np.allclose(np.einsum("ij,ij->" + ("j" if axis == 0 else "i"), o2, o2)
                       / shape[axis], 1.0, rtol=1e-12)
    # and scaling O by c > 0 changes nothing
    o3, _ = mo.normuon_scale(3.5 * o, np.zeros(min(shape)), 0.0, 0.0)
    assert np.allclose(o3, o2, rtol=1e-12)


def test_normuon_two_step_ema():
    m, n = 5, 11
    o1 = rng(3).standard_normal((m, n))
    o2 = rng(4).standard_normal((m, n))
    v0 = rng(5).uniform(0, 1, size=m)
    b = 0.75
    _, v1 = mo.normuon_scale(o1, v0, b, 1e-8)
    _, v2 = mo.normuon_scale(o2, v1, b, 1e-8)
    m1 = np.linalg.norm(o1, axis=1) ** 2 / n
    m2 = np.linalg.norm(o2, axis=1) ** 2 / n
    assert np.allclose(v2, b * b * v0 + b * (1 - b) * m1 + (1 - b) * m2, rtol=1e-13)


def test_normuon_transpose_equivariance():
    o = rng(6).standard_normal((4, 13))
    v0 = rng(7).uniform(0, 1, size=4)
    a, va = mo.normuon_scale(o, v0, 0.9, 1e-6)
    b, vb = mo.normuon_scale(o.T, v0, 0.9, 1e-6)
    assert np.array_equal(va, vb)
    assert np.allclose(a, b.T, rtol=1e-14)


# ------------------------------------------------------- cautious decay
def test_cautious_decay_hand_example():
    # mask = (O*W >= 0): [[1*1 >= 0, 1*-2 < 0], [-1*0.5 < 0, 0*0.4 >= 0]]
    # W' = W - 0.1*O - 0.1*0.5*mask*W, by hand:
    #   [[1 - 0.1 - 0.05, -2 - 0.1], [0.5 + 0.1, 0.4 - 0 - 0.02]]
    w = np.array([[1.0, -2.0], [0.5, 0.4]])
    o = np.array([[1.0, 1.0], [-1.0, 0.0]])
    out = mo.decayed_weight_update(w, o, lr=0.1, scale=1.0, weight_decay=0.5, cautious=True)
    assert np.allclose(out, [[0.85, -2.1], [0.6, 0.38]], rtol=0, atol=1e-15)
    # the sign test is on W before the update: W[0][0] = 1 with O = 20 would
    # change sign after the step but still decays
    out = mo.decayed_weight_update(np.array([[1.0]]), np.array([[20.0]]), 0.1, 1.0, 0.5, True)
    assert np.allclose(out, [[1.0 - 2.0 - 0.05]], rtol=0, atol=1e-15)


def test_decay_special_cases():
    w = rng(8).standard_normal((6, 9))
    o = rng(9).standard_normal((6, 9))
    lr, sc, wd = 0.02, 1.7, 0.1
    plain = mo.weight_update(w, o, lr, sc)
    assert np.array_equal(mo.decayed_weight_update(w, o, lr, sc, 0.0, True), plain)
    assert np.allclose(mo.decayed_weight_update(w, o, lr, sc, wd, False),
                       (1 - lr * wd) * w - lr * sc * o, rtol=1e-14)
    # O with W's signs: every entry decays; O against W's signs: none does
    same = np.abs(o) * np.sign(w)
    assert np.allclose(mo.decayed_weight_update(w, same, lr, sc, wd, True),
                       (1 - lr * wd) * w - lr * sc * same, rtol=1e-14)
    against = -same
    assert np.allclose(mo.decayed_weight_update(w, against, lr, sc, wd, True),
                       w - lr * sc * against, rtol=1e-14)


# ---------------------------------------------------------- the whole step
def test_step_ex_reduces_to_plain_step():
    w = rng(10).standard_normal((8, 24)) * 0.02
    g = rng(11).standard_normal((8, 24))
    b = rng(12).standard_normal((8, 24)) * 1e-3
    w1, b1, o1 = mo.muon_step(w, g, b, 0.95, 0.02, 1.0, QUINTIC)
    r = mo.muon_step_ex(w, g, b, 0.95, 0.02, 1.0, QUINTIC)
    assert np.array_equal(r["w"], w1) and np.array_equal(r["buf"], b1)
    assert np.array_equal(r["o"], o1) and r["v"] is None


def test_step_ex_order_normuon_then_decay():
    # the review's order: orthogonalise, then NorMuon scaling, then the decayed update
    # with the scaled direction; with orthonormal-row NS output the scaling
    # is the closed form of test_normuon_closed_form_on_orthonormal_rows
    m, n = 4, 12
    q = orthonormal_rows(m, n, 13)
    g = q * 7.0  # orthonormal rows scaled: the cubic map drives it to q
    w = rng(14).standard_normal((m, n))
    v0 = np.full(m, 0.01)
    r = mo.muon_step_ex(w, g, np.zeros((m, n)), 0.0, 0.1, 1.0, [wl.CUBIC] * 60,
                        weight_decay=0.3, cautious=True, second_moment=v0,
                        beta2=0.9, normuon_eps=0.0)
    v_expect = 0.9 * 0.01 + 0.1 / n
    assert np.allclose(r["v"], v_expect, rtol=1e-9)
    o_expect = q / math.sqrt(v_expect)
    assert np.allclose(r["o"], o_expect, rtol=1e-8, atol=1e-12)
    mask = o_expect * w >= 0
    assert np.allclose(r["w"], w - 0.1 * o_expect - 0.03 * np.where(mask, w, 0.0), rtol=1e-9)


# ------------------------------------ the pins catch plausible mistakes
def _normuon_mutants():
    def wrong_axis(o, v, beta2, eps):
        o = np.asarray(o, float)
        axis = 1 if o.shape[0] > o.shape[1] else 0
        msq = np.mean(o * o, axis=axis)
        msq = np.resize(msq, np.shape(v))
        nv = beta2 * np.asarray(v) + (1 - beta2) * msq
        d = np.sqrt(nv) + eps
        return o / (d[None, :] if o.shape[0] > o.shape[1] else d[:, None]), nv

    def sum_not_mean(o, v, beta2, eps):
        o = np.asarray(o, float)
        axis = 0 if o.shape[0] > o.shape[1] else 1
        nv = beta2 * np.asarray(v) + (1 - beta2) * np.sum(o * o, axis=axis)
        d = np.sqrt(nv) + eps
        return o / (d[None, :] if axis == 0 else d[:, None]), nv

    def no_sqrt(o, v, beta2, eps):
        o = np.asarray(o, float)
        axis = 0 if o.shape[0] > o.shape[1] else 1
        nv = beta2 * np.asarray(v) + (1 - beta2) * np.mean(o * o, axis=axis)
        d = nv + eps
        return o / (d[None, :] if axis == 0 else d[:, None]), nv

    def swapped_beta(o, v, beta2, eps):
        o = np.asarray(o, float)
        axis = 0 if o.shape[0] > o.shape[1] else 1
        nv = (1 - beta2) * np.asarray(v) + beta2 * np.mean(o * o, axis=axis)
        d = np.sqrt(nv) + eps
        return o / (d[None, :] if axis == 0 else d[:, None]), nv

    return [wrong_axis, sum_not_mean, no_sqrt, swapped_beta]


def _normuon_pins():
    test_normuon_closed_form_on_orthonormal_rows(4, 16)
    test_normuon_tall_uses_columns(16, 4)
    test_normuon_beta2_zero_normalises_rms((3, 7))
    test_normuon_beta2_zero_normalises_rms((7, 3))
    test_normuon_two_step_ema()


@pytest.mark.parametrize("mutant", _normuon_mutants(), ids=lambda f: f.__name__)
def test_planted_normuon_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(mo, "normuon_scale", mutant)
    with pytest.raises(AssertionError):
        _normuon_pins()


def _decay_mutants():
    def strict_mask(w, o, lr, scale, weight_decay, cautious):
        wd = weight_decay
        w = np.asarray(w, float)
        o = np.asarray(o, float)
        mask = (o * w > 0.0) if cautious else np.ones_like(w, dtype=bool)
        return w - lr * scale * o - lr * wd * np.where(mask, w, 0.0)

    def decay_after_update(w, o, lr, scale, weight_decay, cautious):
        wd = weight_decay
        w = np.asarray(w, float)
        o = np.asarray(o, float)
        w1 = w - lr * scale * o
        mask = (o * w1 >= 0.0) if cautious else np.ones_like(w, dtype=bool)
        return w1 - lr * wd * np.where(mask, w1, 0.0)

    def decay_without_lr(w, o, lr, scale, weight_decay, cautious):
        wd = weight_decay
        w = np.asarray(w, float)
        o = np.asarray(o, float)
        mask = (o * w >= 0.0) if cautious else np.ones_like(w, dtype=bool)
        return w - lr * scale * o - wd * np.where(mask, w, 0.0)

    def inverted_mask(w, o, lr, scale, weight_decay, cautious):
        wd = weight_decay
        w = np.asarray(w, float)
        o = np.asarray(o, float)
        mask = (o * w < 0.0) if cautious else np.ones_like(w, dtype=bool)
        return w - lr * scale * o - lr * wd * np.where(mask, w, 0.0)

    return [strict_mask, decay_after_update, decay_without_lr, inverted_mask]


@pytest.mark.parametrize("mutant", _decay_mutants(), ids=lambda f: f.__name__)
def test_planted_decay_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(mo, "decayed_weight_update", mutant)
    with pytest.raises(AssertionError):
        test_cautious_decay_hand_example()
        test_decay_special_cases()


def test_package_exports():
    assert oracle.normuon_scale is mo.normuon_scale
    assert oracle.decayed_weight_update is mo.decayed_weight_update
    assert oracle.muon_step_ex is mo.muon_step_ex
