"""Pins for the merge oracle (CPU only).

* Closed form: if (y0, l0) is itself the softmax-weighted mean and
  log-sum-exp of k values under k logits, merging x under its own logit must
  equal one softmax over all k + 1 values.
* Special cases: l0 = -inf returns x exactly; equal logits average; a very
  low l1 returns y0.
* A small hand-derived example (values written out in the test).
* Central finite differences for gx, gq, gy0 and gl0.
* N-way merge: attention over all keys equals the merge of attention over
  key splits (against the attention oracle); the S = 2 case with the
  logit rho x . q is the residual merge; -inf inputs and rows; finite
  differences.
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


# ------------------------------------------------------ N-way lse merge ----

def test_lse_merge_equals_attention_over_all_keys():
    """Attention over all keys equals the merge of attention over disjoint key
    splits (the identity split-KV attention rests on); the attention oracle is
    an independent computation of the left side."""
    from oracle import attention as oa
    B, H, M, D, c = 1, 2, 7, 5, 0.6
    splits = [3, 1, 6, 4]
    N = sum(splits)
    q, k, v = rand(B, H, M, D), rand(B, H, N, D), rand(B, H, N, D)
    o_all, lse_all = oa.attn_fwd(q, k, v, False, c)
    ys, lses, j = [], [], 0
    for n in splits:
        o_s, l_s = oa.attn_fwd(q, k[:, :, j:j + n], v[:, :, j:j + n], False, c)
        ys.append(o_s.reshape(-1, D))
        lses.append(l_s.reshape(-1))
        j += n
    y, lse = om.lse_merge_fwd(np.stack(ys), np.stack(lses))
    np.testing.assert_allclose(y, o_all.reshape(-1, D), atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, lse_all.reshape(-1), atol=1e-13, rtol=0)


def test_lse_merge_is_the_residual_merge_with_given_logit():
    rows, D, eps = 6, 8, 1e-6
    x, q, y0, l0 = rand(rows, D), rand(D) / 3, rand(rows, D), rand(rows)
    gy, gl = rand(rows, D), rand(rows)
    y_r, lse_r = om.merge_fwd(x, q, y0, l0, eps)
    l1 = (x @ q) / np.sqrt((x * x).mean(axis=1) + eps)
    ys, lses = np.stack([y0, x]), np.stack([l0, l1])
    y, lse = om.lse_merge_fwd(ys, lses)
    np.testing.assert_allclose(y, y_r, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, lse_r, atol=1e-14, rtol=0)
    # the y0 and l0 gradients are the residual merge's gy0 and gl0
    _, _, gy0, gl0 = om.merge_bwd(x, q, y0, l0, gy, gl, eps)
    gys, glses = om.lse_merge_bwd(ys, lses, gy, gl)
    np.testing.assert_allclose(gys[0], gy0, atol=1e-14, rtol=0)
    np.testing.assert_allclose(glses[0], gl0, atol=1e-13, rtol=0)


def test_lse_merge_special_cases():
    S, rows, D = 3, 4, 5
    ys, lses = rand(S, rows, D), rand(S, rows)
    # one input: identity
    y, lse = om.lse_merge_fwd(ys[:1], lses[:1])
    np.testing.assert_array_equal(y, ys[0])
    np.testing.assert_array_equal(lse, lses[0])
    # an input at -inf contributes nothing and gets zero gradients
    l2 = lses.copy()
    l2[1] = -np.inf
    y, lse = om.lse_merge_fwd(ys, l2)
    y_ref, lse_ref = om.lse_merge_fwd(ys[[0, 2]], lses[[0, 2]])
    np.testing.assert_allclose(y, y_ref, atol=1e-15)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-15)
    gys, glses = om.lse_merge_bwd(ys, l2, rand(rows, D), rand(rows))
    assert np.all(gys[1] == 0) and np.all(glses[1] == 0)
    # a row with every input at -inf: y = 0, lse = -inf, zero gradients
    l3 = lses.copy()
    l3[:, 2] = -np.inf
    y, lse = om.lse_merge_fwd(ys, l3)
    assert np.all(y[2] == 0) and np.isneginf(lse[2]) and np.all(np.isfinite(lse[[0, 1, 3]]))
    gys, glses = om.lse_merge_bwd(ys, l3, rand(rows, D), rand(rows))
    assert np.all(gys[:, 2] == 0) and np.all(glses[:, 2] == 0)
    # equal logits average; lse = l + log S
    le = np.broadcast_to(lses[:1], lses.shape).copy()
    y, lse = om.lse_merge_fwd(ys, le)
    np.testing.assert_allclose(y, ys.mean(axis=0), atol=1e-15)
    np.testing.assert_allclose(lse, lses[0] + math.log(S), atol=1e-15)


@pytest.mark.parametrize("with_gl", [True, False])
def test_lse_merge_bwd_finite_differences(with_gl):
    S, rows, D = 3, 2, 4
    ys, lses, gy = rand(S, rows, D), rand(S, rows), rand(rows, D)
    gl = rand(rows) if with_gl else None

    def loss(ys_, lses_):
        y, lse = om.lse_merge_fwd(ys_, lses_)
        return float((y * gy).sum() + (0.0 if gl is None else (lse * gl).sum()))

    def fd(a, f, h=1e-6):
        g = np.zeros_like(a)
        it = np.nditer(a, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            ap, am = a.copy(), a.copy()
            ap[idx] += h
            am[idx] -= h
            g[idx] = (f(ap) - f(am)) / (2 * h)
        return g

    gys, glses = om.lse_merge_bwd(ys, lses, gy, gl)
    np.testing.assert_allclose(gys, fd(ys, lambda a: loss(a, lses)), atol=1e-8, rtol=0)
    np.testing.assert_allclose(glses, fd(lses, lambda a: loss(ys, a)), atol=1e-8, rtol=0)
