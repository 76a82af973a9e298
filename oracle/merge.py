"""fp64 oracle: block-residual two-way online-softmax merge and its VJP.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Source: flash_attn_res 0.1.11, ``slop/backward_phase_2.txt``.  Its
``reference_forward`` is the only statement of the forward; the phase-2 merge
backward kernel recomputes the forward and applies the chain rule.  Shapes:
x, y0 are ``[rows, D]``; the pseudo-query q is ``[D]``; l0 is ``[rows]``.

Per row the forward is
    rho  = (mean_d x_d^2 + eps)^(-1/2)        (inverse RMS of x)
    l1   = rho * (x . q)                      (logit of x against q; no 1/sqrt(D))
    m    = max(l0, l1)
    w0   = exp(l0 - m),  w1 = exp(l1 - m),  Z = w0 + w1
    alpha = w0 / Z,  beta = w1 / Z
    y    = alpha * y0 + beta * x
    lse  = m + log(Z).
l0 = -inf is allowed and gives alpha = 0 exactly (y = x, lse = l1).
"""

import numpy as np


def _forward_terms(x, q, l0, eps):
    D = x.shape[-1]
    rho = 1.0 / np.sqrt((x * x).sum(axis=-1) / D + eps)
    xq = x @ q
    l1 = rho * xq
    m = np.maximum(l0, l1)
    w0 = np.exp(l0 - m)
    w1 = np.exp(l1 - m)
    Z = w0 + w1
    return rho, xq, l1, m, w0 / Z, w1 / Z, Z


def merge_fwd(x, q, y0, l0, eps):
    """Returns (y [rows, D], lse [rows]) as in ``reference_forward``."""
    _, _, _, m, alpha, beta, Z = _forward_terms(x, q, l0, eps)
    y = alpha[:, None] * y0 + beta[:, None] * x
    lse = m + np.log(Z)
    return y, lse


def merge_bwd(x, q, y0, l0, gy, gl, eps):
    """VJP of ``merge_fwd`` for the loss <gy, y> + <gl, lse>.

    Returns (gx [rows, D], gq [D], gy0 [rows, D], gl0 [rows]).  ``gl=None``
    means zeros (the page's launcher does the same).  Derivation, per row:
        d alpha/d l0 = alpha*beta = -d alpha/d l1,  d lse/d l0 = alpha,
        d lse/d l1 = beta,  d l1/d q = rho x,
        d l1/d x = rho q - (x.q) rho^3 x / D      (from d rho/d x = -rho^3 x / D)
    hence, with s = gy . (y0 - x):
        gy0 = alpha gy
        gl0 = alpha gl + alpha beta s
        gl1 = beta gl - alpha beta s
        gx  = beta gy + gl1 (rho q - (x.q) rho^3 x / D)
        gq  = sum over rows of gl1 rho x.
    These are the same terms the page's backward kernel forms."""
    D = x.shape[-1]
    if gl is None:
        gl = np.zeros_like(l0)
    rho, xq, _, _, alpha, beta, _ = _forward_terms(x, q, l0, eps)
    s = (gy * (y0 - x)).sum(axis=-1)
    gy0 = alpha[:, None] * gy
    gl0 = alpha * gl + alpha * beta * s
    gl1 = beta * gl - alpha * beta * s
    dl1_dx = rho[:, None] * q[None, :] - (xq * rho ** 3 / D)[:, None] * x
    gx = beta[:, None] * gy + gl1[:, None] * dl1_dx
    gq = ((gl1 * rho)[:, None] * x).sum(axis=0)
    return gx, gq, gy0, gl0


# ------------------------------------------------- N-way (y, lse) merge ----
#
# The same online-softmax combine with S inputs whose logits are given rather
# than computed from x: the merge of attention partials over key splits
# (split-KV, ring partials).  The residual merge above is its S = 2 case with
# (y_0, l_0) = (y0, l0) and (y_1, l_1) = (x, rho x . q).  Shapes: ys [S, rows,
# D], lses [S, rows]; a row whose S logits are all -inf merges to y = 0 and
# lse = -inf (the convention of an attention row with no visible key).

def lse_merge_fwd(ys, lses):
    """Returns (y [rows, D], lse [rows]):
        lse = log sum_s exp(lse_s),   y = sum_s exp(lse_s - lse) y_s."""
    m = lses.max(axis=0)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    e = np.exp(lses - m_safe[None, :])          # exp(-inf) == 0
    Z = e.sum(axis=0)
    Z_safe = np.where(has, Z, 1.0)
    w = e / Z_safe[None, :]
    y = (w[:, :, None] * ys).sum(axis=0)
    lse = np.where(has, m_safe + np.log(Z_safe), -np.inf)
    return y, lse


def lse_merge_bwd(ys, lses, gy, gl):
    """VJP of ``lse_merge_fwd`` for <gy, y> + <gl, lse>; returns
    (gys [S, rows, D], glses [S, rows]).  With w_s = exp(lse_s - lse):
        d lse / d lse_s = w_s,   d y / d lse_s = w_s (y_s - y),   d y / d y_s = w_s,
    so  gys_s = w_s gy  and  glses_s = w_s (gl + gy . (y_s - y)).
    ``gl=None`` means zeros."""
    y, lse = lse_merge_fwd(ys, lses)
    if gl is None:
        gl = np.zeros_like(lse)
    has = np.isfinite(lse)
    w = np.where(has[None, :], np.exp(lses - np.where(has, lse, 0.0)[None, :]), 0.0)
    gys = w[:, :, None] * gy[None, :, :]
    glses = w * (gl[None, :] + (gy[None, :, :] * (ys - y[None, :, :])).sum(axis=-1))
    return gys, glses
