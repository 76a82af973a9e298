"""GPU parity of the torch autograd / forward-AD wrapper against the fp64 oracle.

Every derivative the wrapper returns comes from the HIP library; these tests
drive it the way a torch user would (``backward`` on both outputs,
``torch.func.jvp``, ``torch.autograd.forward_ad`` dual tensors, a merge
chained after attention) and compare with the oracle's composition of the
same steps.
"""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd.inputs import BF16, F16, F32, AttnWorkload, attn_inputs, draw
from gpu_util import dev, host, log, need_gpu
from tolerance import check_grad, check_lse, check_output

pytestmark = pytest.mark.gpu


def _dense(wl, names=("q", "k", "v", "do")):
    t = attn_inputs(wl, names)
    g = draw(wl.seed + 1, [("g", (wl.B, wl.H, wl.M), 1.0, F32)])["g"]
    return t, g


@pytest.mark.parametrize("case", [(BF16, 1, 2, 256, 256, 128, True), (F16, 1, 2, 150, 77, 64, False),
                                  (F32, 1, 2, 128, 128, 64, True), (BF16, 1, 2, 200, 170, 256, True),
                                  (F16, 1, 2, 130, 190, 16, False)], ids=lambda c: "-".join(map(str, c)))
def test_attention_backward_both_outputs(case):
    torch = need_gpu()
    from attention_fa2_tiles_amd.autograd import attention
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("ag_bwd", dtype, B, H, M, N, D, causal, seed=51 + M)
    log(f"autograd backward {case}")
    t, g = _dense(wl)
    q, k, v = (dev(t[n]).requires_grad_() for n in ("q", "k", "v"))
    o, lse = attention(q, k, v, causal=causal)
    torch.autograd.backward([o, lse], [dev(t["do"]), dev(g)])
    f = {n: t[n].f64 for n in ("q", "k", "v", "do")}
    ro, rl = oracle.attn_fwd(f["q"], f["k"], f["v"], causal, wl.scale())
    rdq, rdk, rdv = oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], causal, wl.scale(), dlse=g.f64)
    check_output("ag.o", host(o), ro, dtype)
    check_lse("ag.lse", host(lse), rl, dtype)
    for n, x, r in (("dq", q, rdq), ("dk", k, rdk), ("dv", v, rdv)):
        assert x.grad.dtype == x.dtype
        check_grad("ag." + n, host(x.grad), r, dtype)


def test_attention_backward_lse_only():
    """Only the LSE output reaches the loss: dO is absent, dV must be 0."""
    torch = need_gpu()
    from attention_fa2_tiles_amd.autograd import attention
    wl = AttnWorkload("ag_lse", BF16, 1, 2, 192, 192, 64, True, seed=57)
    t, g = _dense(wl)
    q, k, v = (dev(t[n]).requires_grad_() for n in ("q", "k", "v"))
    _, lse = attention(q, k, v, causal=True)
    (lse * dev(g)).sum().backward()
    f = {n: t[n].f64 for n in ("q", "k", "v")}
    zero = np.zeros_like(t["do"].f64)
    rdq, rdk, _ = oracle.attn_bwd(f["q"], f["k"], f["v"], zero, True, wl.scale(), dlse=g.f64)
    check_grad("ag_lse.dq", host(q.grad), rdq, BF16)
    check_grad("ag_lse.dk", host(k.grad), rdk, BF16)
    assert np.all(host(v.grad) == 0.0)


JVP_CASES = [(F16, 1, 2, 192, 192, 64, True), (BF16, 1, 2, 150, 100, 128, False), (F32, 1, 2, 128, 192, 64, True),
             (BF16, 1, 2, 160, 224, 256, True), (F16, 1, 2, 192, 96, 16, False)]


@pytest.mark.parametrize("case", JVP_CASES, ids=lambda c: "-".join(map(str, c)))
def test_attention_func_jvp(case):
    torch = need_gpu()
    from attention_fa2_tiles_amd.autograd import attention
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("ag_jvp", dtype, B, H, M, N, D, causal, seed=61 + M)
    log(f"autograd torch.func.jvp {case}")
    names = ("q", "k", "v", "tq", "tk", "tv")
    t = attn_inputs(wl, names)
    d = [dev(t[n]) for n in names]
    (o, lse), (to, tlse) = torch.func.jvp(lambda a, b, c: attention(a, b, c, causal=causal), tuple(d[:3]),
                                          tuple(d[3:]))
    ro, rl, rto, rtl = oracle.attn_fwd_jvp(*[t[n].f64 for n in names], causal, wl.scale())
    check_output("jvp.o", host(o), ro, dtype)
    check_lse("jvp.lse", host(lse), rl, dtype)
    check_grad("jvp.to", host(to), rto, dtype)
    check_grad("jvp.tlse", host(tlse), rtl, dtype)


def test_attention_forward_ad_and_partial_tangents():
    """torch.autograd.forward_ad dual tensors give the same tangents as
    torch.func.jvp, bit for bit (one fused pass each); a tangent on V alone
    leaves the LSE tangent exactly 0."""
    torch = need_gpu()
    import torch.autograd.forward_ad as fwAD
    from attention_fa2_tiles_amd.autograd import attention
    wl = AttnWorkload("ag_dual", F16, 1, 2, 256, 256, 64, True, seed=67)
    names = ("q", "k", "v", "tq", "tk", "tv")
    t = attn_inputs(wl, names)
    d = [dev(t[n]) for n in names]
    _, (to_f, tl_f) = torch.func.jvp(lambda a, b, c: attention(a, b, c, causal=True), tuple(d[:3]), tuple(d[3:]))
    with fwAD.dual_level():
        duals = [fwAD.make_dual(p, tt) for p, tt in zip(d[:3], d[3:])]
        o, lse = attention(*duals, causal=True)
        uo, ul = fwAD.unpack_dual(o), fwAD.unpack_dual(lse)
        assert torch.equal(uo.tangent, to_f) and torch.equal(ul.tangent, tl_f)
        ro, rl, rto, rtl = oracle.attn_fwd_jvp(*[t[n].f64 for n in names], True, wl.scale())
        check_output("dual.o", host(uo.primal), ro, F16)
        check_grad("dual.to", host(uo.tangent), rto, F16)
        check_grad("dual.tlse", host(ul.tangent), rtl, F16)
        # tangent on V only
        o3, l3 = attention(d[0], d[1], fwAD.make_dual(d[2], d[5]), causal=True)
        assert torch.all(fwAD.unpack_dual(l3).tangent == 0)
        z = np.zeros_like(t["q"].f64)
        _, _, rto3, _ = oracle.attn_fwd_jvp(t["q"].f64, t["k"].f64, t["v"].f64, z, np.zeros_like(t["k"].f64),
                                            t["tv"].f64, True, wl.scale())
        check_grad("dual_v.to", host(fwAD.unpack_dual(o3).tangent), rto3, F16)


def test_piecewise_backward_both_outputs():
    torch = need_gpu()
    from attention_fa2_tiles_amd.autograd import piecewise_attention
    wl = AttnWorkload("ag_pw", F16, 1, 2, 200, 170, 64, True, seed=71)
    names = ("q1", "k1", "q2", "k2", "v", "do")
    t = attn_inputs(wl, names)
    g = draw(wl.seed + 1, [("g", (1, 2, 200), 1.0, F32)])["g"]
    x = [dev(t[n]).requires_grad_() for n in names[:5]]
    o, lse = piecewise_attention(*x, 50, causal=True)
    torch.autograd.backward([o, lse], [dev(t["do"]), dev(g)])
    f = [t[n].f64 for n in names]
    ro, rl = oracle.pw_fwd(*f[:5], True, wl.scale(), 50)
    check_output("pw.o", host(o), ro, F16)
    check_lse("pw.lse", host(lse), rl, F16)
    ref = oracle.pw_bwd(*f, True, wl.scale(), 50, dlse=g.f64)
    for n, a, r in zip(("dq1", "dk1", "dq2", "dk2", "dv"), x, ref):
        check_grad("pw." + n, host(a.grad), r, F16)


def test_merge_after_attention():
    """Attention partials (o, lse) merged with a residual stream by the
    two-way online-softmax merge: the merge's LSE gradient reaches the
    attention backward as its dLSE."""
    torch = need_gpu()
    from attention_fa2_tiles_amd.autograd import attention, resmerge
    B, H, M, D = 1, 2, 192, 128
    wl = AttnWorkload("ag_merge", BF16, B, H, M, M, D, True, seed=73)
    t = attn_inputs(wl, ("q", "k", "v"))
    rows = B * H * M
    e = draw(wl.seed + 1, [("x", (rows, D), 1.0, BF16), ("qm", (D,), 1.0 / np.sqrt(D), BF16),
                           ("gy", (rows, D), 1.0, BF16), ("gl", (rows,), 1.0, F32)])
    q, k, v = (dev(t[n]).requires_grad_() for n in ("q", "k", "v"))
    x, qm = dev(e["x"]).requires_grad_(), dev(e["qm"]).requires_grad_()
    o, lse = attention(q, k, v, causal=True)
    y, ly = resmerge(x, qm, o.reshape(rows, D), lse.reshape(rows), eps=1e-6)
    torch.autograd.backward([y, ly], [dev(e["gy"]), dev(e["gl"])])

    f = {n: t[n].f64 for n in ("q", "k", "v")}
    ro, rl = oracle.attn_fwd(f["q"], f["k"], f["v"], True, wl.scale())
    y0, l0 = ro.reshape(rows, D), rl.reshape(rows)
    ry, rly = oracle.merge_fwd(e["x"].f64, e["qm"].f64, y0, l0, 1e-6)
    gx, gqm, gy0, gl0 = oracle.merge_bwd(e["x"].f64, e["qm"].f64, y0, l0, e["gy"].f64, e["gl"].f64, 1e-6)
    rdq, rdk, rdv = oracle.attn_bwd(f["q"], f["k"], f["v"], gy0.reshape(B, H, M, D), True, wl.scale(),
                                    dlse=gl0.reshape(B, H, M))
    check_output("chain.y", host(y), ry, BF16)
    check_lse("chain.lse", host(ly), rly, BF16)
    for n, a, r in (("gx", x, gx), ("gq", qm, gqm), ("dq", q, rdq), ("dk", k, rdk), ("dv", v, rdv)):
        check_grad("chain." + n, host(a.grad), r, BF16)
