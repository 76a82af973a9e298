"""fp64 oracle: scaled-dot-product attention, its backward, its forward-mode
JVP, and piecewise attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it.

Conventions (shared by every function here)
-------------------------------------------
* Tensors are numpy float64 arrays, ``q``-like ``[B, H, M, D]`` and ``k``-like
  ``[B, H, N, D]``.  Each (b, h) head is independent and is computed on its own,
  whole: the full M x N score matrix of a head is formed, so no sum over keys
  or queries is split into blocks.
* ``sm_scale`` is used literally (the library maps its own "0 = default" flag
  to 1/sqrt(D); the oracle never does).
* Causal masking is aligned bottom-right: query i sees key j iff
  ``j <= i + (N - M)``.  This is how FlagAttention ``piecewise.py`` offsets
  queries by ``P_SEQ = N - M`` in ``_fwd_kernel`` and the backward kernels; for
  M == N it is the usual lower-triangular mask of the gist's ``test_op``.
* A row with no visible key has O = 0 and LSE = -inf (FlagAttention
  ``_fwd_kernel``, the empty-line branch of its epilogue).
* LSE is the natural-log log-sum-exp of the scaled scores (FlagAttention
  ``_fwd_kernel`` epilogue).  The gist stores a base-2 value instead; the two
  differ by a factor ln 2 and carry the same information.
"""

import numpy as np

NEG_INF = -np.inf


def allowed_mask(M, N, causal):
    """Boolean [M, N]: True where key j is visible to query i.

    Bottom-right causal alignment, as in FlagAttention ``piecewise.py``
    (``causal_mask = P_SEQ + i >= j`` with ``P_SEQ = N - M``)."""
    if not causal:
        return np.ones((M, N), dtype=bool)
    i = np.arange(M)[:, None]
    j = np.arange(N)[None, :]
    return j <= i + (N - M)


def near_mask(M, N, w):
    """Boolean [M, N]: True where piecewise attention uses the (q1, k1) pair.

    The query-key distance is ``dist(i, j) = i + (N - M) - j`` (the same
    bottom-right offset as the causal mask).  The docstring of FlagAttention's
    ``attention()`` says the first pair is used while the distance is not
    greater than the threshold, and the second pair otherwise; this oracle
    takes that prose, on the absolute distance, as the rule:
    near  <=>  |dist| <= w.  (The page's kernels select the second pair when
    ``P_SEQ + i >= j + w``, i.e. dist >= w; that rule equals this one with w
    shifted by one on the causal side.  The reading is recorded with the
    other readings of the pages in the design notes.)"""
    i = np.arange(M)[:, None]
    j = np.arange(N)[None, :]
    dist = i + (N - M) - j
    return np.abs(dist) <= w


def _softmax_rows(S, A):
    """Row softmax of the scores S restricted to the visible set A.

    Returns (P, lse): P is zero outside A; a row with no visible key gets
    P = 0 and lse = -inf."""
    Sm = np.where(A, S, NEG_INF)
    m = Sm.max(axis=1)
    has = np.isfinite(m)
    m_safe = np.where(has, m, 0.0)
    E = np.exp(Sm - m_safe[:, None])  # exp(-inf) == 0 outside A
    Z = E.sum(axis=1)
    Z_safe = np.where(has, Z, 1.0)
    P = E / Z_safe[:, None]
    lse = np.where(has, m_safe + np.log(Z_safe), NEG_INF)
    return P, lse


def _scores(q, k, sm_scale):
    return sm_scale * (q @ k.T)


def attn_probs(q, k, causal, sm_scale):
    """Softmax probabilities P [B, H, M, N] and LSE [B, H, M].

    P_ij = exp(S_ij - LSE_i) on the visible set and 0 elsewhere, with
    S = sm_scale * Q K^T (the gist's ``test_op`` reference: scaled matmul,
    causal -inf fill, softmax in full precision)."""
    B, H, M, _ = q.shape
    N = k.shape[2]
    A = allowed_mask(M, N, causal)
    P = np.zeros((B, H, M, N))
    lse = np.zeros((B, H, M))
    for b in range(B):
        for h in range(H):
            P[b, h], lse[b, h] = _softmax_rows(_scores(q[b, h], k[b, h], sm_scale), A)
    return P, lse


def attn_fwd(q, k, v, causal, sm_scale):
    """Attention forward: returns (O [B,H,M,D], LSE [B,H,M]).

    O = softmax(sm_scale * Q K^T) V with the causal mask applied before the
    softmax; this is the computation the gist's ``_attn_fwd`` kernel tiles
    with an online softmax, and the same plain definition its ``test_op``
    checks against."""
    P, lse = attn_probs(q, k, causal, sm_scale)
    o = np.einsum("bhmn,bhnd->bhmd", P, v)
    return o, lse


def attn_bwd(q, k, v, do, causal, sm_scale, dlse=None):
    """Attention backward: returns (dQ, dK, dV) for the loss <dO, O> + <dLSE, LSE>.

    The analytic vector-Jacobian product that the gist's backward computes by
    recomputation (``_attn_bwd_preprocess`` for Delta, ``_attn_bwd_dkdv`` and
    ``_attn_bwd_dq``), here evaluated on whole matrices:
        dV = P^T dO
        dP = dO V^T
        Delta_i = sum_d O_id dO_id
        dS = P * (dP - Delta)
        dQ = sm_scale * dS K,   dK = sm_scale * dS^T Q.
    Masking is the same for causal and non-causal; the non-causal case visits
    every block (the correction proposed in the gist's comment thread).

    ``dlse`` ([B, H, M], optional, zeros when None) is the gradient reaching
    the log-sum-exp output, as the residual merge's backward hands to its
    LSE inputs.  The gist's backward has no such input; by the chain rule,
    dLSE_i / dS_ij = P_ij, so it adds P * dLSE to dS:
        dS = P * (dP - (Delta - dLSE))."""
    B, H, M, D = q.shape
    N = k.shape[2]
    A = allowed_mask(M, N, causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            P, _ = _softmax_rows(_scores(q[b, h], k[b, h], sm_scale), A)
            O = P @ v[b, h]
            dO = do[b, h]
            dv[b, h] = P.T @ dO
            dP = dO @ v[b, h].T
            delta = (O * dO).sum(axis=1)
            if dlse is not None:
                delta = delta - dlse[b, h]
            dS = P * (dP - delta[:, None])
            dq[b, h] = sm_scale * (dS @ k[b, h])
            dk[b, h] = sm_scale * (dS.T @ q[b, h])
    return dq, dk, dv


def attn_fwd_jvp(q, k, v, tq, tk, tv, causal, sm_scale):
    """Forward-mode JVP of attention: returns (O, LSE, tO, tLSE).

    The directional derivative of O along (tQ, tK, tV), as the gist's fused
    forward accumulates it (the ``ENABLE_JVP`` branch of ``_attn_fwd_inner``
    and the tangent epilogue of ``_attn_fwd``; method of Lu and Song,
    arXiv 2410.11081):
        Sdot = sm_scale * (tQ K^T + Q tK^T), zero on masked entries
        mu_i = sum_j P_ij Sdot_ij
        tO   = (P * Sdot) V - mu O + P tV.
    The gist returns no tangent for LSE; since dLSE_i / dS_ij = P_ij it is
        tLSE = mu
    (natural log units; 0 for a row with no visible key)."""
    B, H, M, D = q.shape
    N = k.shape[2]
    A = allowed_mask(M, N, causal)
    o = np.zeros_like(q)
    lse = np.zeros((B, H, M))
    to = np.zeros_like(q)
    tlse = np.zeros((B, H, M))
    for b in range(B):
        for h in range(H):
            P, lse[b, h] = _softmax_rows(_scores(q[b, h], k[b, h], sm_scale), A)
            O = P @ v[b, h]
            Sdot = sm_scale * (tq[b, h] @ k[b, h].T + q[b, h] @ tk[b, h].T)
            Sdot = np.where(A, Sdot, 0.0)
            PS = P * Sdot
            mu = PS.sum(axis=1)
            o[b, h] = O
            to[b, h] = PS @ v[b, h] - mu[:, None] * O + P @ tv[b, h]
            tlse[b, h] = mu
    return o, lse, to, tlse


def _pw_scores(q1, k1, q2, k2, near, sm_scale):
    return sm_scale * np.where(near, q1 @ k1.T, q2 @ k2.T)


def pw_fwd(q1, k1, q2, k2, v, causal, sm_scale, w):
    """Piecewise attention forward: returns (O, LSE).

    FlagAttention ``piecewise.py`` (``_fwd_kernel``): the score of (i, j) is
    sm_scale * q1_i . k1_j for near pairs and sm_scale * q2_i . k2_j for the
    rest (``near_mask``); after that the softmax and P V are those of
    ``attn_fwd``."""
    B, H, M, D = q1.shape
    N = k1.shape[2]
    A = allowed_mask(M, N, causal)
    near = near_mask(M, N, w)
    o = np.zeros_like(q1)
    lse = np.zeros((B, H, M))
    for b in range(B):
        for h in range(H):
            S = _pw_scores(q1[b, h], k1[b, h], q2[b, h], k2[b, h], near, sm_scale)
            P, lse[b, h] = _softmax_rows(S, A)
            o[b, h] = P @ v[b, h]
    return o, lse


def pw_bwd(q1, k1, q2, k2, v, do, causal, sm_scale, w, dlse=None):
    """Piecewise attention backward: returns (dq1, dk1, dq2, dk2, dv).

    FlagAttention ``piecewise.py`` (``_bwd_kv_kernel``, ``_bwd_q_kernel``):
    dS is formed as in ``attn_bwd`` and split by the near mask; the near part
    flows to (q1, k1) and the far part to (q2, k2):
        dq1 = c (dS*near) k1,   dk1 = c (dS*near)^T q1,
        dq2 = c (dS*far)  k2,   dk2 = c (dS*far)^T  q2,   dv = P^T dO.
    ``dlse`` enters dS as in ``attn_bwd``."""
    B, H, M, D = q1.shape
    N = k1.shape[2]
    A = allowed_mask(M, N, causal)
    near = near_mask(M, N, w)
    far = ~near
    dq1 = np.zeros_like(q1)
    dk1 = np.zeros_like(k1)
    dq2 = np.zeros_like(q2)
    dk2 = np.zeros_like(k2)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            S = _pw_scores(q1[b, h], k1[b, h], q2[b, h], k2[b, h], near, sm_scale)
            P, _ = _softmax_rows(S, A)
            O = P @ v[b, h]
            dO = do[b, h]
            dv[b, h] = P.T @ dO
            dP = dO @ v[b, h].T
            delta = (O * dO).sum(axis=1)
            if dlse is not None:
                delta = delta - dlse[b, h]
            dS = P * (dP - delta[:, None])
            dSn = np.where(near, dS, 0.0)
            dSf = np.where(far, dS, 0.0)
            dq1[b, h] = sm_scale * (dSn @ k1[b, h])
            dk1[b, h] = sm_scale * (dSn.T @ q1[b, h])
            dq2[b, h] = sm_scale * (dSf @ k2[b, h])
            dk2[b, h] = sm_scale * (dSf.T @ q2[b, h])
    return dq1, dk1, dq2, dk2, dv
