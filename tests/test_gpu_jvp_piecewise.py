"""GPU parity: fa_fwd_jvp (O, LSE and both tangents), pw_fwd and pw_bwd (with
and without a gradient reaching LSE) against the fp64 oracle."""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16, F16, F32, PIECEWISE_W, WORKLOADS, AttnWorkload, attn_inputs, draw
from gpu_util import check_guards, dev, empty_f32, filled, guarded, guarded_f32, host, log, need_gpu
from tolerance import check_grad, check_lse, check_output

pytestmark = pytest.mark.gpu

JVP_NAMES = ("q", "k", "v", "tq", "tk", "tv")
PW_NAMES = ("q1", "k1", "q2", "k2", "v", "do")


# ------------------------------------------------------------------ JVP ----

def run_jvp(wl, t):
    torch = need_gpu()
    q, k, v, tq, tk, tv = (dev(t[n]) for n in JVP_NAMES)
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o = guarded((B, H, M, D), wl.dtype)
    to = guarded((B, H, M, D), wl.dtype)
    lse = guarded_f32((B, H, M))
    tlse = guarded_f32((B, H, M))
    lib.fa_fwd_jvp_tlse(wl.dtype, q, k, v, tq, tk, tv, o, lse, to, tlse, B, H, M, N, D, wl.causal, wl.sm_scale)
    torch.cuda.synchronize()
    res = {"o": host(o), "lse": host(lse), "to": host(to), "tlse": host(tlse)}
    check_guards()
    return res


def compare_jvp(wl, t, got, heads=None):
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)] if heads is None else heads
    for (b, h) in pairs:
        f = [t[n].f64[b:b + 1, h:h + 1] for n in JVP_NAMES]
        o, lse, to, tlse = oracle.attn_fwd_jvp(*f, wl.causal, wl.scale())
        tag = f"{wl.name}[b={b},h={h}]"
        check_output(f"{tag}.o", got["o"][b, h], o[0, 0], wl.dtype)
        check_lse(f"{tag}.lse", got["lse"][b, h], lse[0, 0], wl.dtype)
        check_grad(f"{tag}.to", got["to"][b, h], to[0, 0], wl.dtype)
        check_grad(f"{tag}.tlse", got["tlse"][b, h], tlse[0, 0], wl.dtype)


JVP_SMALL = [
    (F16, 2, 2, 192, 192, 64, True),
    (F16, 2, 2, 192, 192, 64, False),
    (BF16, 1, 2, 128, 256, 128, True),
    (F16, 1, 2, 256, 128, 128, True),
    (F32, 1, 2, 128, 128, 64, False),
    (F32, 1, 2, 128, 192, 128, True),
    (F16, 1, 2, 100, 150, 64, True),      # ragged lengths
    (BF16, 1, 2, 150, 100, 128, False),
    (F16, 1, 2, 150, 100, 32, True),      # head dims 32 and (fp32) 256
    (BF16, 2, 2, 128, 128, 32, False),
    (F32, 1, 1, 64, 80, 256, True),
]


@pytest.mark.parametrize("case", JVP_SMALL, ids=lambda c: "-".join(map(str, c)))
def test_jvp_small(case):
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("jvp_small", dtype, B, H, M, N, D, causal, seed=21 + M + D)
    log(f"jvp small parity {case}")
    t = attn_inputs(wl, JVP_NAMES)
    compare_jvp(wl, t, run_jvp(wl, t))


def test_jvp_forward_part_matches_fa_fwd():
    """O and LSE from the fused JVP pass equal those of fa_fwd."""
    torch = need_gpu()
    wl = AttnWorkload("jvp_vs_fwd", F16, 1, 2, 256, 256, 64, True, seed=3)
    t = attn_inputs(wl, JVP_NAMES)
    got = run_jvp(wl, t)
    q, k, v = (dev(t[n]) for n in ("q", "k", "v"))
    o = filled((1, 2, 256, 64), F16)
    lse = empty_f32((1, 2, 256))
    lib.fa_fwd(F16, q, k, v, o, lse, 1, 2, 256, 256, 64, 1, 0.0)
    torch.cuda.synchronize()
    np.testing.assert_allclose(got["o"], host(o), atol=2e-3, rtol=0)
    np.testing.assert_allclose(got["lse"], host(lse), atol=1e-5, rtol=0)


@pytest.mark.parametrize("name", ["jvp_f16_b4h16_s1024_d64_causal", "jvp_f16_b4h16_s1024_d64"])
def test_jvp_full_size(name):
    wl = WORKLOADS[name]
    log(f"jvp full-size {name}")
    t = attn_inputs(wl, JVP_NAMES)
    compare_jvp(wl, t, run_jvp(wl, t), heads=[(0, 0), (2, 7), (3, 15)])


# ------------------------------------------------------------ piecewise ----

def run_pw(wl, t, w, with_bwd=True, dlse=None):
    torch = need_gpu()
    q1, k1, q2, k2, v, do = (dev(t[n]) for n in PW_NAMES)
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o = guarded((B, H, M, D), wl.dtype)
    lse = guarded_f32((B, H, M))
    lib.pw_fwd(wl.dtype, q1, k1, q2, k2, v, o, lse, B, H, M, N, D, wl.causal, wl.sm_scale, w)
    out = {"o": o, "lse": lse}
    if with_bwd:
        grads = {n: guarded(x.shape, wl.dtype) for n, x in
                 (("dq1", q1), ("dk1", k1), ("dq2", q2), ("dk2", k2), ("dv", v))}
        nb = lib.pw_bwd_workspace_size(B, H, M, N, D, wl.dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        gl = [grads[n] for n in ("dq1", "dk1", "dq2", "dk2", "dv")]
        if dlse is None:
            lib.pw_bwd(wl.dtype, q1, k1, q2, k2, v, o, do, lse, *gl, ws, nb, B, H, M, N, D, wl.causal,
                       wl.sm_scale, w)
        else:
            lib.pw_bwd_dlse(wl.dtype, q1, k1, q2, k2, v, o, do, lse, dlse, *gl, ws, nb, B, H, M, N, D,
                            wl.causal, wl.sm_scale, w)
        out.update(grads)
    torch.cuda.synchronize()
    res = {kk: host(vv) for kk, vv in out.items()}
    check_guards()
    return res


def compare_pw(wl, t, got, w, heads=None, with_bwd=True, dlse=None):
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)] if heads is None else heads
    c = wl.scale()
    for (b, h) in pairs:
        f = [t[n].f64[b:b + 1, h:h + 1] for n in PW_NAMES]
        o, lse = oracle.pw_fwd(*f[:5], wl.causal, c, w)
        tag = f"{wl.name}[w={w},b={b},h={h}]"
        check_output(f"{tag}.o", got["o"][b, h], o[0, 0], wl.dtype)
        check_lse(f"{tag}.lse", got["lse"][b, h], lse[0, 0], wl.dtype)
        if with_bwd:
            g = None if dlse is None else dlse[b:b + 1, h:h + 1]
            ref = oracle.pw_bwd(*f, wl.causal, c, w, dlse=g)
            for n, r in zip(("dq1", "dk1", "dq2", "dk2", "dv"), ref):
                check_grad(f"{tag}.{n}", got[n][b, h], r[0, 0], wl.dtype)


PW_SMALL = [
    # dtype, B, H, M, N, D, causal, w
    (F16, 1, 2, 256, 256, 64, True, 100),      # band edge inside blocks
    (F16, 1, 2, 256, 256, 64, False, 100),     # |dist| <= w on both sides
    (F16, 1, 2, 256, 256, 64, True, 64),       # band edge on a block edge
    (BF16, 1, 2, 192, 320, 128, True, 37),     # M != N
    (F16, 1, 2, 256, 256, 64, True, -1),       # every pair far
    (F16, 1, 2, 256, 256, 64, False, 1000),    # every pair near
    (F16, 1, 2, 256, 256, 64, True, 0),        # only the diagonal is near
    (F16, 1, 2, 640, 704, 64, True, 150),      # several workgroups, M != N
    (BF16, 2, 2, 512, 448, 64, False, 90),     # M > N, both signs of dist
    (F16, 1, 2, 333, 517, 64, True, 77),       # ragged, several workgroups
    (F16, 1, 2, 190, 333, 64, False, 70),      # ragged, partial key block first
    (BF16, 1, 2, 300, 200, 64, True, 40),      # M > N: rows with no visible key
    (F32, 1, 2, 128, 128, 64, True, 20),
    (F32, 1, 2, 128, 192, 128, False, 50),
    (F16, 1, 2, 200, 170, 64, True, 50),       # ragged lengths
    (BF16, 1, 2, 130, 250, 128, False, 60),
    (F16, 1, 2, 200, 170, 32, True, 50),       # head dims 32 and (fp32) 256
    (BF16, 1, 2, 256, 256, 32, False, 100),
    (F32, 1, 1, 64, 96, 256, True, 20),
]


@pytest.mark.parametrize("case", PW_SMALL, ids=lambda c: "-".join(map(str, c)))
def test_pw_small(case):
    dtype, B, H, M, N, D, causal, w = case
    wl = AttnWorkload("pw_small", dtype, B, H, M, N, D, causal, seed=31 + M + (w % 97))
    log(f"pw small parity {case}")
    t = attn_inputs(wl, PW_NAMES)
    compare_pw(wl, t, run_pw(wl, t, w), w)


@pytest.mark.parametrize("case", [(F16, 1, 2, 256, 256, 64, True, 100), (BF16, 1, 2, 130, 250, 128, False, 60),
                                  (F32, 1, 2, 128, 128, 64, True, 20)], ids=lambda c: "-".join(map(str, c)))
def test_pw_lse_gradient(case):
    dtype, B, H, M, N, D, causal, w = case
    wl = AttnWorkload("pw_dlse", dtype, B, H, M, N, D, causal, seed=41 + M)
    log(f"pw lse-gradient parity {case}")
    t = attn_inputs(wl, PW_NAMES)
    g = draw(wl.seed + 1, [("dlse", (B, H, M), 1.0, F32)])["dlse"]
    compare_pw(wl, t, run_pw(wl, t, w, dlse=dev(g)), w, dlse=g.f64)


def test_pw_full_size():
    wl = WORKLOADS["piecewise_f16_b2h16_s4096_d64_w1024"]
    log("pw full-size")
    t = attn_inputs(wl, PW_NAMES)
    got = run_pw(wl, t, PIECEWISE_W)
    compare_pw(wl, t, got, PIECEWISE_W, heads=[(0, 3), (1, 14)])
