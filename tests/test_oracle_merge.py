"""Pins for the merge oracle (CPU only).

* Closed form: if (y0, l0) is itself the softmax-weighted mean and
  log-sum-exp of k values under k logits, merging x under its own logit must
  equal one softmax over all k + 1 values.
* Special cases: l0 = -inf returns x exactly; equal logits average; a very
  low l1 returns y0.
* A small hand-derived example (values written out in the test).
* Central finite differences for gx, gq, gy0 and gl0.
"""

import math

import numpy as np
import pytest

from oracle import merge as om

RNG = np.random.default_rng(7)


def rand(*shape):
    return RNG.standard_normal(shape)


def test_closed_form_softmax_merge():
    rows, D, kk, eps = 5, 16, 4, 1e-6
    x, q = rand(rows, D), rand(D) / 4
    vals = rand(rows, kk, D)
    logits = rand(rows, kk)
    m0 = logits.max(1)
    w = np.exp(logits - m0[:, None])
    y0 = (w[:, :, None] * vals).sum(1) / w.sum(1)[:, None]
    l0 = m0 + np.log(w.sum(1))
    y, lse = om.merge_fwd(x, q, y0, l0, eps)
    rho = 1 / np.sqrt((x ** 2).mean(1) + eps)
    l1 = rho * (x @ q)
    all_logits = np.concatenate([logits, l1[:, None]], 1)
    all_vals = np.concatenate([vals, x[:, None, :]], 1)
    mm = all_logits.max(1)
    ww = np.exp(all_logits - mm[:, None])
    np.testing.assert_allclose(y, (ww[:, :, None] * all_vals).sum(1) / ww.sum(1)[:, None], atol=1e-13)
    np.testing.assert_allclose(lse, mm + np.log(ww.sum(1)), atol=1e-13)


def test_special_cases():
    rows, D, eps = 4, 8, 1e-6
    x, q, y0 = rand(rows, D), rand(D), rand(rows, D)
    l0 = np.full(rows, -np.inf)
    y, lse = om.merge_fwd(x, q, y0, l0, eps)
    rho = 1 / np.sqrt((x ** 2).mean(1) + eps)
    assert np.array_equal(y, x)
    np.testing.assert_allclose(lse, rho * (x @ q), atol=1e-15)
    gx, gq, gy0, gl0 = om.merge_bwd(x, q, y0, l0, rand(rows, D), rand(rows), eps)
    assert np.all(gy0 == 0) and np.all(gl0 == 0)
    # l1 far below l0 -> y = y0
    y, lse = om.merge_fwd(x, q, y0, np.full(rows, 1e4), eps)
    np.testing.assert_allclose(y, y0, atol=1e-15)
    np.testing.assert_allclose(lse, 1e4, atol=0)


def test_hand_example():
    """x = (1, -1), q = (1, 0), eps = 0: mean(x^2) = 1 so rho = 1 and
    l1 = x . q = 1.  With l0 = 1 both weights are 1/2, so y = (y0 + x)/2 and
    lse = 1 + ln 2.  Backward with gy = (1, 0), gl = 0: gy0 = (1/2, 0);
    s = gy . (y0 - x) = 3 - 1 = 2; gl0 = alpha beta s = 1/2; gl1 = -1/2;
    d l1/d x = q - (x.q) x / 2 = (1/2, 1/2); gx = beta gy + gl1 (1/2, 1/2)
    = (1/4, -1/4); gq = gl1 rho x = (-1/2, 1/2)."""
    x = np.array([[1.0, -1.0]])
    q = np.array([1.0, 0.0])
    y0 = np.array([[3.0, 5.0]])
    l0 = np.array([1.0])
    y, lse = om.merge_fwd(x, q, y0, l0, 0.0)
    np.testing.assert_allclose(y, [[2.0, 2.0]], atol=1e-15)
    np.testing.assert_allclose(lse, [1.0 + math.log(2.0)], atol=1e-15)
    gx, gq, gy0, gl0 = om.merge_bwd(x, q, y0, l0, np.array([[1.0, 0.0]]), None, 0.0)
    np.testing.assert_allclose(gy0, [[0.5, 0.0]], atol=1e-15)
    np.testing.assert_allclose(gl0, [0.5], atol=1e-15)
    np.testing.assert_allclose(gx, [[0.25, -0.25]], atol=1e-15)
    np.testing.assert_allclose(gq, [-0.5, 0.5], atol=1e-15)


@pytest.mark.parametrize("with_gl", [True, False])
def test_bwd_finite_differences(with_gl):
    rows, D, eps = 3, 6, 1e-3
    x, q, y0, l0 = rand(rows, D), rand(D), rand(rows, D), rand(rows)
    gy = rand(rows, D)
    gl = rand(rows) if with_gl else None

    def loss(x_, q_, y0_, l0_):
        y, lse = om.merge_fwd(x_, q_, y0_, l0_, eps)
        val = float((y * gy).sum())
        if gl is not None:
            val += float((lse * gl).sum())
        return val

    def fd(i, a, h=1e-6):
        g = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            argsp = [x, q, y0, l0]
            argsm = [x, q, y0, l0]
            argsp[i] = ap
            argsm[i] = am
            g[idx] = (loss(*argsp) - loss(*argsm)) / (2 * h)
        return g

    gx, gq, gy0, gl0 = om.merge_bwd(x, q, y0, l0, gy, gl, eps)
    for i, g in enumerate((gx, gq, gy0, gl0)):
        ref = fd(i, [x, q, y0, l0][i])
        np.testing.assert_allclose(g, ref, atol=1e-8 * max(1.0, np.abs(ref).max()), rtol=0)
