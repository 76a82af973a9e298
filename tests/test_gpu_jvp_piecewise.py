"""GPU parity: fa_fwd_jvp (O, LSE and both tangents), pw_fwd and pw_bwd (with
and without a gradient reaching LSE) against the fp64 oracle."""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import (BF16, F16, F32, PIECEWISE_W, WORKLOADS, AttnWorkload, Draw, Tensor,
                                            attn_inputs, draw, to_storage)
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
    (F16, 1, 2, 100, 120, 16, True),      # head dim 16: the D = 32 kernels over zero-padded rows
    (BF16, 1, 1, 64, 64, 16, False),
    (BF16, 2, 2, 384, 256, 16, True),     # M > N, several workgroups
    (F32, 1, 2, 70, 90, 16, False),       # fp32 head dim 16: the generic kernels
    (F16, 1, 2, 90, 70, 256, True),       # 16-bit 256: output columns split over two workgroups
    (BF16, 1, 1, 64, 96, 256, False),
    (BF16, 2, 2, 256, 256, 256, True),
    (F16, 1, 2, 384, 384, 256, False),
    (BF16, 1, 2, 300, 170, 256, True),    # M > N: rows that see no key
    (F16, 1, 1, 130, 450, 256, False),
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
    # the fp16 JVP rescales at every new row maximum (P <= 1) while fa_fwd lets
    # P reach 2^8: each rounds P to fp16 (relative error <= 2^-11) at its own
    # scale before summing it, so the two LSEs agree to within 2 * 2^-11
    np.testing.assert_allclose(got["lse"], host(lse), atol=2.0 ** -10, rtol=0)


@pytest.mark.parametrize("name", ["jvp_f16_b4h16_s1024_d64_causal", "jvp_f16_b4h16_s1024_d64"])
def test_jvp_full_size(name):
    wl = WORKLOADS[name]
    log(f"jvp full-size {name}")
    t = attn_inputs(wl, JVP_NAMES)
    compare_jvp(wl, t, run_jvp(wl, t))  # every head


@pytest.mark.parametrize("D", [256, 16])
def test_jvp_head_dims_bench_shape_sampled_heads(D):
    """The fused JVP at the head-dim workloads the benchmark times (causal
    bf16 B1 H16 2048^2, D = 256 and 16): three heads against the oracle."""
    wl = AttnWorkload(f"jvp_causal_bf16_b1h16_s2048_d{D}", BF16, 1, 16, 2048, 2048, D, True, seed=6)
    log(f"jvp head-dim bench shape D = {D}")
    t = attn_inputs(wl, JVP_NAMES)
    got = run_jvp(wl, t)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values"
    compare_jvp(wl, t, got, heads=[(0, 0), (0, 7), (0, 15)])


def ramp_tangent_inputs(M, N, D, dtype, seed):
    """Scores that stay flat over the first 64 keys and then rise by almost
    8 (log2 units) towards the last key, with tangent scores near 300: an
    online softmax that lets P grow to 2^8 before rescaling would form
    P * Sdot near 7e4, above the fp16 range."""
    rng = np.random.default_rng(seed)
    c, log2e = 1.0 / np.sqrt(D), 1.4426950408889634
    q = (0.05 * rng.standard_normal((1, 1, M, D))).astype(np.float32)
    k = (0.05 * rng.standard_normal((1, 1, N, D))).astype(np.float32)
    q[..., 0] = 4.0
    j = np.arange(N)
    k[0, 0, :, 0] = np.where(j < 64, 0.0, 7.9 * (j - 64) / (N - 65)) / (c * log2e * 4.0)
    tk = np.zeros((1, 1, N, D), np.float32)
    tk[..., 0] = (75.0 / c) * np.where(rng.standard_normal(N) > 0, 1.0, -1.0)  # tangent scores +-300
    arrays = {"q": q, "k": k, "v": rng.standard_normal((1, 1, N, D)).astype(np.float32),
              "tq": rng.standard_normal((1, 1, M, D)).astype(np.float32), "tk": tk,
              "tv": rng.standard_normal((1, 1, N, D)).astype(np.float32)}
    out = Draw(seed)
    for n in JVP_NAMES:
        st, f = to_storage(arrays[n], dtype)
        out.tensors[n] = Tensor(n, st, f, dtype)
    return out


@pytest.mark.parametrize("D", [64, 256])
def test_jvp_large_tangent_fp16(D):
    """fp16 JVP whose later keys raise the row maximum by almost 8 (log2)
    while the tangent scores are near 300: the tangent output stays finite
    and meets the bar."""
    wl = AttnWorkload("jvp_ramp", F16, 1, 1, 256, 256, D, False, seed=5)
    log(f"jvp large tangents, fp16, D = {D}")
    t = ramp_tangent_inputs(256, 256, D, F16, seed=5)
    got = run_jvp(wl, t)
    assert np.all(np.isfinite(got["to"])), "tangent output overflowed"
    f = [t[n].f64 for n in JVP_NAMES]
    assert np.abs(wl.scale() * np.einsum("bhmd,bhnd->bhmn", f[0], f[4])).max() > 256
    compare_jvp(wl, t, got)


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
    (F16, 1, 2, 100, 130, 16, True, 30),      # head dim 16: the D = 32 kernels over zero-padded rows
    (BF16, 1, 1, 96, 64, 16, False, 20),
    (BF16, 1, 2, 512, 448, 16, True, 70),     # several workgroups, M > N
    (F32, 1, 1, 80, 70, 16, True, 15),        # fp32 head dim 16: the generic kernels
    (BF16, 1, 2, 90, 110, 256, True, 25),     # 16-bit 256: the generic kernels
    (F16, 1, 1, 64, 64, 256, False, 10),
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


@pytest.mark.parametrize("case", [(F16, 2, 2, 1024, 1024, 64, True), (BF16, 1, 2, 384, 320, 128, False),
                                  (BF16, 1, 2, 256, 256, 256, True)], ids=lambda c: "-".join(map(str, c)))
def test_jvp_deterministic(case):
    """Two fused-JVP runs on the same inputs give bitwise-equal outputs."""
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("jvp_det", dtype, B, H, M, N, D, causal, seed=51 + M + D)
    log(f"jvp determinism {case}")
    t = attn_inputs(wl, JVP_NAMES)
    a, b = run_jvp(wl, t), run_jvp(wl, t)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_pw_deterministic():
    """Two piecewise forward + backward runs give bitwise-equal outputs."""
    wl = AttnWorkload("pw_det", F16, 1, 2, 640, 704, 64, True, seed=61)
    log("pw determinism")
    t = attn_inputs(wl, PW_NAMES)
    a, b = run_pw(wl, t, 150), run_pw(wl, t, 150)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


_PW_FULL = {}


@pytest.mark.parametrize("chunk", range(4))
def test_pw_full_size(chunk):
    """fp16 B2 H16 4096 D64 causal, w = 1024: every head against the oracle
    (O, LSE and the five gradients), in four chunks of 8 heads; the GPU runs
    once."""
    wl = WORKLOADS["piecewise_f16_b2h16_s4096_d64_w1024"]
    if "run" not in _PW_FULL:
        log("pw full-size: GPU run")
        t = attn_inputs(wl, PW_NAMES)
        _PW_FULL["run"] = (t, run_pw(wl, t, PIECEWISE_W))
    t, got = _PW_FULL["run"]
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    heads = pairs[chunk * 8:(chunk + 1) * 8]
    log(f"pw full-size heads {heads[0]}..{heads[-1]}")
    compare_pw(wl, t, got, PIECEWISE_W, heads=heads)
    if chunk == 3:
        _PW_FULL.clear()
