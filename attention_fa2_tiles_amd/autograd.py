"""torch autograd and forward-mode AD over the C ABI.

Thin glue in the spirit of the tutorial's ``JVPAttn`` Function (its
``forward``, ``backward``, ``jvp`` and ``fwd_dual``): every value is computed
by the HIP library through ``attention_fa2_tiles_amd.lib``; this module only
allocates outputs and workspaces with torch, makes operands contiguous and
routes gradients and tangents to the right entry point.  There is no CPU or
PyTorch fallback: a tensor that is not on the GPU, or a missing library,
raises.

Functions
---------
``attention(q, k, v, causal=False, sm_scale=None) -> (o, lse)``
    Plain inputs: fa_fwd.  Dual inputs (``torch.autograd.forward_ad`` or
    ``torch.func.jvp``): one fused fa_fwd_jvp pass gives o, lse and both
    tangents (the tutorial's ``fwd_dual``: the tangents are unpacked and
    passed to the Function next to the dual primals).  Reverse mode: fa_bwd
    with the gradients of both outputs (the LSE gradient enters dS as
    P * dLSE).
``piecewise_attention(q1, k1, q2, k2, v, w, causal=False, sm_scale=None)``
    pw_fwd / pw_bwd (reverse mode only; the pages give no piecewise JVP).
``resmerge(x, q, y0, l0, eps=1e-6) -> (y, lse)``
    resmerge_fwd / resmerge_bwd (reverse mode).  Chained after
    ``attention`` (y0 = its o rows, l0 = its lse), the merge's LSE gradient
    flows into the attention backward as its dLSE.

Layouts are those of ``include/fa.h``: q-like [B, H, M, D], k-like
[B, H, N, D], lse [B, H, M] float32; merge rows [rows, D], l0 and lse
[rows] float32, q [D].  ``sm_scale=None`` selects 1/sqrt(D).
"""

import torch
import torch.autograd.forward_ad as fwAD

from . import lib

_CODES = {torch.float32: lib.F32, torch.float16: lib.F16, torch.bfloat16: lib.BF16}


def _code(t):
    if t.dtype not in _CODES:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, float16 or bfloat16")
    if not t.is_cuda:
        raise RuntimeError("the HIP attention library needs GPU tensors (there is no CPU path)")
    return _CODES[t.dtype]


def _scale(sm_scale):
    return 0.0 if sm_scale is None else float(sm_scale)


def _attn_shape(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("expected q [B,H,M,D] and k, v [B,H,N,D]")
    B, H, M, D = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != D:
        raise ValueError("q and k disagree on B, H or D")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    return B, H, M, k.shape[2], D


def _c(t):
    return t.contiguous()


def _zeros_or(t, like):
    return torch.zeros_like(like) if t is None else _c(t)


def _fwd(q, k, v, causal, sm_scale):
    B, H, M, N, D = _attn_shape(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    lib.fa_fwd(_code(q), q, k, v, o, lse, B, H, M, N, D, int(causal), _scale(sm_scale))
    return o, lse


def _fwd_jvp(q, k, v, tq, tk, tv, causal, sm_scale):
    B, H, M, N, D = _attn_shape(q, k, v)
    o, to = torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, M), dtype=torch.float32, device=q.device)
    tlse = torch.empty_like(lse)
    lib.fa_fwd_jvp_tlse(_code(q), q, k, v, tq, tk, tv, o, lse, to, tlse, B, H, M, N, D, int(causal),
                   _scale(sm_scale))
    return o, lse, to, tlse


class _Attention(torch.autograd.Function):
    # The tangents travel as extra inputs: forward runs the fused JVP pass when
    # they are present and saves the output tangents, and the jvp rule hands
    # them back.  Under torch.func.jvp the jvp rule only sees wrapped tensors
    # without storage, so no kernel could run there.
    @staticmethod
    def forward(q, k, v, tq, tk, tv, causal, sm_scale):
        q, k, v = _c(q), _c(k), _c(v)
        if tq is None and tk is None and tv is None:
            o, lse = _fwd(q, k, v, causal, sm_scale)
            return o, lse, None, None
        tq, tk, tv = _zeros_or(tq, q), _zeros_or(tk, k), _zeros_or(tv, v)
        return _fwd_jvp(q, k, v, tq, tk, tv, causal, sm_scale)

    @staticmethod
    def setup_context(ctx, inputs, output):
        q, k, v, _, _, _, causal, sm_scale = inputs
        o, lse, to, tlse = output
        ctx.causal, ctx.sm_scale = causal, sm_scale
        ctx.set_materialize_grads(False)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.has_tangents = to is not None
        if to is not None:
            # outputs only as a carrier: torch asks for their tangents, not their gradients
            ctx.mark_non_differentiable(to, tlse)
            ctx.save_for_forward(to, tlse)

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, do, dlse, _dto, _dtlse):
        q, k, v, o, lse = ctx.saved_tensors
        q, k, v = _c(q), _c(k), _c(v)
        B, H, M, N, D = _attn_shape(q, k, v)
        do = _zeros_or(do, o)
        dlse = None if dlse is None else _c(dlse).float()
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        nb = lib.fa_bwd_workspace_size(B, H, M, N, D, _code(q))
        ws = torch.empty(nb, dtype=torch.uint8, device=q.device)
        lib.fa_bwd_dlse(_code(q), q, k, v, o, do, lse, dlse, dq, dk, dv, ws, nb, B, H, M, N, D,
                        int(ctx.causal), _scale(ctx.sm_scale))
        return dq, dk, dv, None, None, None, None, None

    @staticmethod
    def jvp(ctx, *_tangents):
        if not ctx.has_tangents:
            raise RuntimeError("forward-mode derivatives need the tangents at call time; call attention() "
                               "on the dual tensors")
        to, tlse = ctx.saved_tensors
        return to, tlse, None, None


def attention(q, k, v, causal=False, sm_scale=None):
    """Attention forward (o, lse) with reverse- and forward-mode derivatives.

    With dual inputs (torch.autograd.forward_ad or torch.func.jvp), one fused
    fa_fwd_jvp pass computes o, lse and their tangents; otherwise fa_fwd
    runs.  Reverse mode runs fa_bwd with the gradients of both outputs."""
    tans = [fwAD.unpack_dual(t).tangent for t in (q, k, v)]
    # The dual inputs themselves make torch call the jvp rule; the tangents
    # also go in separately because forward receives primals only.
    o, lse, _, _ = _Attention.apply(q, k, v, *tans, bool(causal), sm_scale)
    return o, lse


class _Piecewise(torch.autograd.Function):
    @staticmethod
    def forward(q1, k1, q2, k2, v, w, causal, sm_scale):
        q1, k1, q2, k2, v = (_c(t) for t in (q1, k1, q2, k2, v))
        B, H, M, N, D = _attn_shape(q1, k1, v)
        if q2.shape != q1.shape or k2.shape != k1.shape or q2.dtype != q1.dtype or k2.dtype != k1.dtype:
            raise ValueError("q2, k2 must match q1, k1")
        o = torch.empty_like(q1)
        lse = torch.empty((B, H, M), dtype=torch.float32, device=q1.device)
        lib.pw_fwd(_code(q1), q1, k1, q2, k2, v, o, lse, B, H, M, N, D, int(causal), _scale(sm_scale), int(w))
        return o, lse

    @staticmethod
    def setup_context(ctx, inputs, output):
        q1, k1, q2, k2, v, w, causal, sm_scale = inputs
        o, lse = output
        ctx.w, ctx.causal, ctx.sm_scale = w, causal, sm_scale
        ctx.set_materialize_grads(False)
        ctx.save_for_backward(q1, k1, q2, k2, v, o, lse)

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, do, dlse):
        q1, k1, q2, k2, v, o, lse = ctx.saved_tensors
        q1, k1, q2, k2, v = (_c(t) for t in (q1, k1, q2, k2, v))
        B, H, M, N, D = _attn_shape(q1, k1, v)
        do = _zeros_or(do, o)
        dlse = None if dlse is None else _c(dlse).float()
        g = [torch.empty_like(t) for t in (q1, k1, q2, k2, v)]
        nb = lib.pw_bwd_workspace_size(B, H, M, N, D, _code(q1))
        ws = torch.empty(nb, dtype=torch.uint8, device=q1.device)
        lib.pw_bwd_dlse(_code(q1), q1, k1, q2, k2, v, o, do, lse, dlse, *g, ws, nb, B, H, M, N, D,
                        int(ctx.causal), _scale(ctx.sm_scale), int(ctx.w))
        return (*g, None, None, None)


def piecewise_attention(q1, k1, q2, k2, v, w, causal=False, sm_scale=None):
    """Piecewise attention forward (o, lse): pairs with |distance| <= w score
    with (q1, k1), the rest with (q2, k2); reverse mode through pw_bwd."""
    return _Piecewise.apply(q1, k1, q2, k2, v, int(w), bool(causal), sm_scale)


class _ResMerge(torch.autograd.Function):
    @staticmethod
    def forward(x, q, y0, l0, eps):
        x, q, y0, l0 = _c(x), _c(q), _c(y0), _c(l0)
        if x.dim() != 2 or y0.shape != x.shape or q.shape != (x.shape[1],) or l0.shape != (x.shape[0],):
            raise ValueError("expected x, y0 [rows, D], q [D], l0 [rows]")
        if l0.dtype != torch.float32 or not (x.dtype == q.dtype == y0.dtype):
            raise TypeError("x, q, y0 share a dtype; l0 is float32")
        rows, D = x.shape
        y = torch.empty_like(x)
        lse = torch.empty((rows,), dtype=torch.float32, device=x.device)
        lib.resmerge_fwd(_code(x), x, q, y0, l0, y, lse, rows, D, float(eps))
        return y, lse

    @staticmethod
    def setup_context(ctx, inputs, output):
        x, q, y0, l0, eps = inputs
        ctx.eps = eps
        ctx.set_materialize_grads(False)
        ctx.save_for_backward(x, q, y0, l0)

    @staticmethod
    @torch.autograd.function.once_differentiable
    def backward(ctx, gy, gl):
        x, q, y0, l0 = (_c(t) for t in ctx.saved_tensors)
        rows, D = x.shape
        gy = _zeros_or(gy, x)
        gl = None if gl is None else _c(gl).float()
        gx, gy0 = torch.empty_like(x), torch.empty_like(y0)
        gq = torch.empty((D,), dtype=torch.float32, device=x.device)
        gl0 = torch.empty((rows,), dtype=torch.float32, device=x.device)
        nb = lib.resmerge_bwd_workspace_size(rows, D)
        ws = torch.empty(nb, dtype=torch.uint8, device=x.device)
        lib.resmerge_bwd(_code(x), x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, ws, nb, rows, D, float(ctx.eps))
        # gq is accumulated in float32; autograd casts it to q's dtype
        return gx, gq, gy0, gl0, None


def resmerge(x, q, y0, l0, eps=1e-6):
    """Block-residual two-way merge (y, lse) with reverse mode through
    resmerge_bwd."""
    return _ResMerge.apply(x, q, y0, l0, float(eps))
