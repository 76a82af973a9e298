"""Pins for the piecewise-attention oracle (CPU only).

* Reductions to ordinary attention, itself pinned to torch SDPA: a threshold
  covering every distance makes every pair near (result = attention on
  (q1, k1)); a negative threshold makes every pair far (attention on
  (q2, k2)); q2 = q1, k2 = k1 gives plain attention and dq1 + dq2 = dq.
* A hand-built closed form that decides the boundary dist == w.
* Central finite differences for all five gradients.
"""

import math

import numpy as np
import pytest

from oracle import attention as oa

RNG = np.random.default_rng(99)


def rand(*shape):
    return RNG.standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_reduces_to_attention(causal):
    M = N = 12
    D = 4
    q1, k1, q2, k2, v, do = (rand(1, 2, M, D) for _ in range(6))
    c = 0.45
    o_near, l_near = oa.pw_fwd(q1, k1, q2, k2, v, causal, c, w=M + N)
    o_ref, l_ref = oa.attn_fwd(q1, k1, v, causal, c)
    np.testing.assert_allclose(o_near, o_ref, atol=1e-14)
    np.testing.assert_allclose(l_near, l_ref, atol=1e-14)
    o_far, l_far = oa.pw_fwd(q1, k1, q2, k2, v, causal, c, w=-1)
    o_ref2, l_ref2 = oa.attn_fwd(q2, k2, v, causal, c)
    np.testing.assert_allclose(o_far, o_ref2, atol=1e-14)
    np.testing.assert_allclose(l_far, l_ref2, atol=1e-14)
    # gradients in the two limits
    dq1, dk1, dq2, dk2, dv = oa.pw_bwd(q1, k1, q2, k2, v, do, causal, c, w=M + N)
    rq, rk, rv = oa.attn_bwd(q1, k1, v, do, causal, c)
    np.testing.assert_allclose(dq1, rq, atol=1e-13)
    np.testing.assert_allclose(dk1, rk, atol=1e-13)
    np.testing.assert_allclose(dv, rv, atol=1e-13)
    assert np.all(dq2 == 0) and np.all(dk2 == 0)
    dq1, dk1, dq2, dk2, dv = oa.pw_bwd(q1, k1, q2, k2, v, do, causal, c, w=-1)
    rq, rk, rv = oa.attn_bwd(q2, k2, v, do, causal, c)
    np.testing.assert_allclose(dq2, rq, atol=1e-13)
    np.testing.assert_allclose(dk2, rk, atol=1e-13)
    np.testing.assert_allclose(dv, rv, atol=1e-13)
    assert np.all(dq1 == 0) and np.all(dk1 == 0)
    # identical pairs: plain attention, and the split gradients add up
    for w in (0, 3, 7):
        o, _ = oa.pw_fwd(q1, k1, q1, k1, v, causal, c, w)
        ro, _ = oa.attn_fwd(q1, k1, v, causal, c)
        np.testing.assert_allclose(o, ro, atol=1e-14)
        dq1, dk1, dq2, dk2, dv = oa.pw_bwd(q1, k1, q1, k1, v, do, causal, c, w)
        rq, rk, rv = oa.attn_bwd(q1, k1, v, do, causal, c)
        np.testing.assert_allclose(dq1 + dq2, rq, atol=1e-13)
        np.testing.assert_allclose(dk1 + dk2, rk, atol=1e-13)
        np.testing.assert_allclose(dv, rv, atol=1e-13)


def test_boundary_closed_form():
    """M = N = 4, w = 1, non-causal, scale 1.  q1 . k1 = 0 for every pair and
    q2 . k2 = L for every pair, so S_ij = 0 when |i - j| <= 1 and L otherwise.
    Row i then weighs its near keys by 1 and its far keys by e^L.  With
    v_j = e_j (one-hot values) O_i is exactly that weight vector normalised;
    a pair at distance exactly 1 = w must count as near."""
    M = N = 4
    L = math.log(3.0)
    q1 = np.zeros((1, 1, M, 2))
    k1 = np.ones((1, 1, N, 2))
    q2 = np.tile(np.array([L, 0.0]), (1, 1, M, 1))
    k2 = np.tile(np.array([1.0, 5.0]), (1, 1, N, 1))
    v = np.eye(N).reshape(1, 1, N, N)
    # v has D = N; the scores use D = 2, so pad q/k to D = 4 with zeros
    pad = np.zeros((1, 1, M, 2))
    q1, k1, q2, k2 = (np.concatenate([a, pad], axis=-1) for a in (q1, k1, q2, k2))
    o, lse = oa.pw_fwd(q1, k1, q2, k2, v, False, 1.0, w=1)
    for i in range(M):
        wts = np.array([1.0 if abs(i - j) <= 1 else 3.0 for j in range(N)])
        np.testing.assert_allclose(o[0, 0, i], wts / wts.sum(), atol=1e-15)
        assert abs(lse[0, 0, i] - math.log(wts.sum())) < 1e-14
    # with w = 0 only the diagonal is near
    o, _ = oa.pw_fwd(q1, k1, q2, k2, v, False, 1.0, w=0)
    for i in range(M):
        wts = np.array([1.0 if i == j else 3.0 for j in range(N)])
        np.testing.assert_allclose(o[0, 0, i], wts / wts.sum(), atol=1e-15)


def test_near_mask_reading():
    """Pin the reading: near <=> |i + (N - M) - j| <= w."""
    nm = oa.near_mask(3, 5, 1)
    expect = np.array([[abs(i + 2 - j) <= 1 for j in range(5)] for i in range(3)])
    assert np.array_equal(nm, expect)
    assert not oa.near_mask(4, 4, -1).any()
    assert oa.near_mask(4, 4, 3).all()


def _fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("with_lse", [False, True])
def test_bwd_finite_differences(causal, with_lse):
    """Loss <dO, O> (+ <g, LSE> when with_lse) against central differences."""
    M = N = 6
    D, c, w = 3, 0.7, 2
    q1, k1, q2, k2, v, do = (rand(1, 1, M, D) for _ in range(6))
    gl = rand(1, 1, M) if with_lse else np.zeros((1, 1, M))
    grads = oa.pw_bwd(q1, k1, q2, k2, v, do, causal, c, w, dlse=gl if with_lse else None)
    args = [q1, k1, q2, k2, v]

    def loss_with(idx, x):
        a = list(args)
        a[idx] = x
        o, lse = oa.pw_fwd(*a, causal, c, w)
        return float((o * do).sum() + (lse * gl).sum())

    for idx, g in enumerate(grads):
        fd = _fd_grad(lambda x: loss_with(idx, x), args[idx])
        np.testing.assert_allclose(g, fd, atol=1e-8 * max(1.0, np.abs(fd).max()), rtol=0)
