"""Pins for the fp64 attention oracle (CPU only).

Each test ties ``oracle.attention`` to something other than itself:
  * torch's CPU float64 ``scaled_dot_product_attention`` (math backend), its
    autograd and its forward-mode AD -- an independent library routine;
  * a pure-Python brute-force loop on tiny shapes;
  * central finite differences of the oracle's own forward (pins the backward
    and the JVP to the forward);
  * invariants and closed forms (softmax rows sum to 1, constant V rows,
    first causal row, zero scale, translation invariance in keys).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention import SDPBackend, sdpa_kernel

from oracle import attention as oa

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a))


def _sdpa(q, k, v, causal, scale, M, N):
    """torch SDPA in float64 on the CPU with a bottom-right causal mask."""
    mask = None
    if causal:
        i = torch.arange(M)[:, None]
        j = torch.arange(N)[None, :]
        mask = j <= i + (N - M)
    with sdpa_kernel(SDPBackend.MATH):
        return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


# ----------------------------------------------------------------- forward --

def _brute_fwd(q, k, v, causal, c):
    """Scalar triple loop with math.fsum; independent of numpy's matmul."""
    B, H, M, D = q.shape
    N = k.shape[2]
    o = [[[[0.0] * D for _ in range(M)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * M for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(M):
                js = [j for j in range(N) if (not causal) or j <= i + N - M]
                if not js:
                    lse[b][h][i] = -math.inf
                    continue
                s = {j: c * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) for j in js}
                mx = max(s.values())
                z = math.fsum(math.exp(s[j] - mx) for j in js)
                lse[b][h][i] = mx + math.log(z)
                for d in range(D):
                    o[b][h][i][d] = math.fsum(math.exp(s[j] - lse[b][h][i]) * v[b, h, j, d] for j in js)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N", [(5, 5), (3, 6), (6, 4), (1, 1), (1, 7)])
def test_fwd_brute_force(causal, M, N):
    q, k, v = rand(1, 2, M, 3), rand(1, 2, N, 3), rand(1, 2, N, 3)
    o, lse = oa.attn_fwd(q, k, v, causal, 0.7)
    ob, lb = _brute_fwd(q, k, v, causal, 0.7)
    np.testing.assert_allclose(o, ob, atol=1e-12, rtol=0)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    fin = np.isfinite(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N,D", [(16, 16, 8), (8, 24, 16), (33, 33, 4)])
def test_fwd_vs_torch_sdpa(causal, M, N, D):
    q, k, v = rand(2, 3, M, D), rand(2, 3, N, D), rand(2, 3, N, D)
    o, lse = oa.attn_fwd(q, k, v, causal, 0.3)
    ref = _sdpa(_t(q), _t(k), _t(v), causal, 0.3, M, N).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12, rtol=0)
    # LSE against torch.logsumexp of the masked library scores
    s = 0.3 * torch.matmul(_t(q), _t(k).transpose(-1, -2).contiguous())
    if causal:
        i = torch.arange(M)[:, None]
        j = torch.arange(N)[None, :]
        s = s.masked_fill(~(j <= i + (N - M)), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12, rtol=0)


def test_fwd_invariants():
    M = N = 12
    D = 5
    q, k = rand(1, 1, M, D), rand(1, 1, N, D)
    for causal in (False, True):
        P, lse = oa.attn_probs(q, k, causal, 0.4)
        np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
        # LSE equals the log-sum-exp of the visible scores (math.fsum)
        A = oa.allowed_mask(M, N, causal)
        for i in range(M):
            s = [0.4 * float(q[0, 0, i] @ k[0, 0, j]) for j in range(N) if A[i, j]]
            assert abs(lse[0, 0, i] - math.log(math.fsum(math.exp(x) for x in s))) < 1e-12
        # constant V rows give O = that row
        u = rand(D)
        v = np.broadcast_to(u, (1, 1, N, D)).copy()
        o, _ = oa.attn_fwd(q, k, v, causal, 0.4)
        np.testing.assert_allclose(o[0, 0], np.broadcast_to(u, (M, D)), atol=1e-13)
    # first causal row sees only key 0
    v = rand(1, 1, N, D)
    o, lse = oa.attn_fwd(q, k, v, True, 0.4)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.4 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14
    # zero scale: O is the mean of the visible values, LSE = log |A(i)|
    for causal in (False, True):
        o, lse = oa.attn_fwd(q, k, v, causal, 0.0)
        A = oa.allowed_mask(M, N, causal)
        for i in range(M):
            np.testing.assert_allclose(o[0, 0, i], v[0, 0, A[i]].mean(0), atol=1e-14)
            assert abs(lse[0, 0, i] - math.log(A[i].sum())) < 1e-14
    # a single key gives O = v0
    o, _ = oa.attn_fwd(rand(1, 1, 1, D), rand(1, 1, 1, D), v[:, :, :1], False, 0.4)
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, 0], atol=1e-15)


def test_fwd_empty_rows():
    """Causal with M > N: the first M-N rows see no key -> O = 0, LSE = -inf."""
    q, k, v = rand(1, 1, 6, 3), rand(1, 1, 4, 3), rand(1, 1, 4, 3)
    o, lse = oa.attn_fwd(q, k, v, True, 0.5)
    assert np.all(o[0, 0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(np.isfinite(lse[0, 0, 2:]))
    # the remaining rows are ordinary attention over keys 0..i-2
    o2, _ = oa.attn_fwd(q[:, :, 2:], k, v, True, 0.5)
    np.testing.assert_allclose(o[0, 0, 2:], o2[0, 0], atol=1e-15)


# ---------------------------------------------------------------- backward --

def _loss(q, k, v, do, causal, c):
    o, _ = oa.attn_fwd(q, k, v, causal, c)
    return float((o * do).sum())


def _fd_grad(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        xp = x.copy()
        xm = x.copy()
        xp[idx] += h
        xm[idx] -= h
        g[idx] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N", [(5, 5), (3, 5)])
def test_bwd_finite_differences(causal, M, N):
    D, c = 3, 0.8
    q, k, v, do = rand(1, 1, M, D), rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, M, D)
    dq, dk, dv = oa.attn_bwd(q, k, v, do, causal, c)
    gq = _fd_grad(lambda x: _loss(x, k, v, do, causal, c), q)
    gk = _fd_grad(lambda x: _loss(q, x, v, do, causal, c), k)
    gv = _fd_grad(lambda x: _loss(q, k, x, do, causal, c), v)
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(a, b, atol=1e-8 * max(1.0, np.abs(b).max()), rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_vs_torch_autograd(causal):
    M = N = 24
    D = 8
    q, k, v, do = rand(2, 2, M, D), rand(2, 2, N, D), rand(2, 2, N, D), rand(2, 2, M, D)
    tq, tk, tv = (_t(a).requires_grad_() for a in (q, k, v))
    o = _sdpa(tq, tk, tv, causal, 0.35, M, N)
    o.backward(_t(do))
    dq, dk, dv = oa.attn_bwd(q, k, v, do, causal, 0.35)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=0)


def test_bwd_noncausal_keys_before_queries():
    """Non-causal dK of an early key must receive contributions from later
    query rows *and* earlier ones; a backward that only walks the causal band
    (the defect discussed in the gist's comment thread) gets dK wrong.  Here
    we check the oracle is not band-limited: changing a query row that lies
    after the key changes that key's gradient in both modes, but changing a
    query row before the key changes it only when non-causal."""
    M = N = 6
    D = 4
    q, k, v, do = rand(1, 1, M, D), rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, M, D)
    key = 3
    for causal, expect_change in ((False, True), (True, False)):
        _, dk, _ = oa.attn_bwd(q, k, v, do, causal, 0.5)
        q2 = q.copy()
        q2[0, 0, 1] += 1.0  # query row 1 < key 3
        _, dk2, _ = oa.attn_bwd(q2, k, v, do, causal, 0.5)
        changed = not np.allclose(dk[0, 0, key], dk2[0, 0, key], atol=1e-14)
        assert changed == expect_change


def test_bwd_invariants():
    M = N = 10
    D = 4
    q, k, v, do = rand(1, 2, M, D), rand(1, 2, N, D), rand(1, 2, N, D), rand(1, 2, M, D)
    for causal in (False, True):
        dq, dk, dv = oa.attn_bwd(q, k, v, do, causal, 0.6)
        # shifting every key by the same vector leaves O unchanged -> sum_j dK_j = 0
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        # softmax rows sum to one -> sum_j dV_j = sum_i dO_i
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    # causal row 0 is v0 regardless of q0 -> dQ_0 = 0
    dq, _, _ = oa.attn_bwd(q, k, v, do, True, 0.6)
    np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-15)


def _loss_lse(q, k, v, do, g, causal, c):
    o, lse = oa.attn_fwd(q, k, v, causal, c)
    return float((o * do).sum() + (lse * g).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("M,N", [(5, 5), (3, 5)])
def test_bwd_lse_gradient_finite_differences(causal, M, N):
    """A gradient reaching LSE (loss <dO, O> + <g, LSE>) against central
    differences of the forward."""
    D, c = 3, 0.7
    q, k, v, do = rand(1, 1, M, D), rand(1, 1, N, D), rand(1, 1, N, D), rand(1, 1, M, D)
    g = rand(1, 1, M)
    dq, dk, dv = oa.attn_bwd(q, k, v, do, causal, c, dlse=g)
    gq = _fd_grad(lambda x: _loss_lse(x, k, v, do, g, causal, c), q)
    gk = _fd_grad(lambda x: _loss_lse(q, x, v, do, g, causal, c), k)
    gv = _fd_grad(lambda x: _loss_lse(q, k, x, do, g, causal, c), v)
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(a, b, atol=1e-8 * max(1.0, np.abs(b).max()), rtol=0)


def test_bwd_lse_gradient_closed_forms():
    M = N = 7
    D, c = 4, 0.6
    q, k, v = rand(1, 2, M, D), rand(1, 2, N, D), rand(1, 2, N, D)
    g = rand(1, 2, M)
    zero_do = np.zeros_like(q)
    for causal in (False, True):
        dq, dk, dv = oa.attn_bwd(q, k, v, zero_do, causal, c, dlse=g)
        np.testing.assert_allclose(dv, 0.0, atol=0)  # LSE does not depend on V
        # moving every key by u moves LSE_i by c q_i . u, so sum_j dK_j = c sum_i g_i q_i
        np.testing.assert_allclose(dk.sum(axis=2), c * np.einsum("bhm,bhmd->bhd", g, q), atol=1e-12)
        # scaling Q by (1 + t) scales every score, dLSE_i/dt = sum_j P_ij S_ij
        P, _ = oa.attn_probs(q, k, causal, c)
        S = c * np.einsum("bhmd,bhnd->bhmn", q, k)
        lhs = float((dq * q).sum())
        rhs = float((g * (P * np.where(P > 0, S, 0.0)).sum(axis=3)).sum())
        assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(rhs))
    # g = 0 is the plain backward
    do = rand(1, 2, M, D)
    a = oa.attn_bwd(q, k, v, do, True, c, dlse=np.zeros((1, 2, M)))
    b = oa.attn_bwd(q, k, v, do, True, c)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


# --------------------------------------------------------------------- JVP --

@pytest.mark.parametrize("causal", [False, True])
def test_jvp_vs_torch_func_jvp(causal):
    M = N = 20
    D = 8
    args = [rand(1, 3, M, D), rand(1, 3, N, D), rand(1, 3, N, D)]
    tans = [rand(1, 3, M, D), rand(1, 3, N, D), rand(1, 3, N, D)]
    o, lse, to, tlse = oa.attn_fwd_jvp(*args, *tans, causal, 0.25)

    def f(a, b, c):
        return _sdpa(a, b, c, causal, 0.25, M, N)

    def f_lse(a, b):
        # torch's logsumexp of the masked scaled scores (independent of P)
        s = 0.25 * (a @ b.transpose(-1, -2))
        if causal:
            i = torch.arange(M)[:, None]
            j = torch.arange(N)[None, :]
            s = s.masked_fill(j > i + (N - M), -math.inf)
        return torch.logsumexp(s, dim=-1)

    with sdpa_kernel(SDPBackend.MATH):
        p, t = torch.func.jvp(f, tuple(_t(a) for a in args), tuple(_t(a) for a in tans))
    np.testing.assert_allclose(o, p.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(to, t.numpy(), atol=1e-12, rtol=0)
    pl, tl = torch.func.jvp(f_lse, (_t(args[0]), _t(args[1])), (_t(tans[0]), _t(tans[1])))
    np.testing.assert_allclose(lse, pl.numpy(), atol=1e-12, rtol=0)
    np.testing.assert_allclose(tlse, tl.numpy(), atol=1e-12, rtol=0)
    o2, lse2 = oa.attn_fwd(*args, causal, 0.25)
    np.testing.assert_allclose(o, o2, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, lse2, atol=1e-14, rtol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_jvp_directional_fd_and_adjoint(causal):
    M, N, D, c = 6, 6, 4, 0.9
    q, k, v = rand(1, 1, M, D), rand(1, 1, N, D), rand(1, 1, N, D)
    tq, tk, tv = rand(1, 1, M, D), rand(1, 1, N, D), rand(1, 1, N, D)
    _, _, to, tlse = oa.attn_fwd_jvp(q, k, v, tq, tk, tv, causal, c)
    h = 1e-6
    op, lp = oa.attn_fwd(q + h * tq, k + h * tk, v + h * tv, causal, c)
    om, lm = oa.attn_fwd(q - h * tq, k - h * tk, v - h * tv, causal, c)
    np.testing.assert_allclose(to, (op - om) / (2 * h), atol=1e-8, rtol=0)
    np.testing.assert_allclose(tlse, (lp - lm) / (2 * h), atol=1e-8, rtol=0)
    # <dO, tO> = <dQ, tQ> + <dK, tK> + <dV, tV> ties the JVP to the VJP
    do = rand(1, 1, M, D)
    dq, dk, dv = oa.attn_bwd(q, k, v, do, causal, c)
    lhs = float((do * to).sum())
    rhs = float((dq * tq).sum() + (dk * tk).sum() + (dv * tv).sum())
    assert abs(lhs - rhs) < 1e-12 * max(1.0, abs(lhs))


def test_jvp_special_cases():
    M = N = 8
    D = 4
    q, k, v = rand(1, 2, M, D), rand(1, 2, N, D), rand(1, 2, N, D)
    z_q, z_k = np.zeros_like(q), np.zeros_like(k)
    for causal in (False, True):
        o, _, to, tlse = oa.attn_fwd_jvp(q, k, v, z_q, z_k, v, causal, 0.5)
        np.testing.assert_allclose(to, o, atol=1e-14)  # O is linear in V
        np.testing.assert_allclose(tlse, 0.0, atol=0)  # LSE does not depend on V
        u = rand(D)
        tk = np.broadcast_to(u, k.shape).copy()  # every key moves by u
        _, _, to, tlse = oa.attn_fwd_jvp(q, k, v, z_q, tk, z_k, causal, 0.5)
        np.testing.assert_allclose(to, 0.0, atol=1e-13)
        # every score of row i moves by 0.5 q_i . u, so LSE_i moves by as much
        np.testing.assert_allclose(tlse, 0.5 * (q @ u), atol=1e-13)
        vc = np.broadcast_to(rand(D), v.shape).copy()  # constant V, no V tangent
        _, _, to, _ = oa.attn_fwd_jvp(q, k, vc, rand(*q.shape), rand(*k.shape), z_k, causal, 0.5)
        np.testing.assert_allclose(to, 0.0, atol=1e-13)
    # causal with M > N: rows with no visible key have a zero LSE tangent
    q3 = rand(1, 1, 9, D)
    k3, v3 = rand(1, 1, 4, D), rand(1, 1, 4, D)
    _, lse, _, tlse = oa.attn_fwd_jvp(q3, k3, v3, rand(*q3.shape), rand(*k3.shape), rand(*v3.shape), True, 0.5)
    assert np.all(np.isneginf(lse[..., :5])) and np.all(tlse[..., :5] == 0.0)
    assert np.all(tlse[..., 5:] != 0.0)
