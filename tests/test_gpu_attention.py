"""GPU parity: fa_fwd / fa_bwd (and its three steps) against the fp64 oracle.

Small shapes are compared element by element on every output; they span
several tiles in both directions, a half-filled last query block, M != N
(bottom-right causal alignment, including query rows that see no key),
lengths that are not tile multiples (down to a single score), both head dims
and all three dtypes, with guard regions around every output.  The full-size workloads (causal bf16
B4 H16 2048 D128 and non-causal bf16 B1 H32 8192 D128) run in the same launch
configuration the benchmark times and are compared on whole sampled heads.
"""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16, F16, F32, WORKLOADS, AttnWorkload, attn_inputs, draw
from gpu_util import check_guards, dev, empty_f32, filled, guarded, guarded_f32, host, log, need_gpu
from tolerance import check_fp32_abs, check_grad, check_lse, check_output

pytestmark = pytest.mark.gpu


def run_fwd_bwd(wl, t, with_bwd=True, steps=False, guard=False, dlse=None):
    torch = need_gpu()
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    alloc = guarded if guard else filled
    o = alloc((B, H, M, D), wl.dtype)
    lse = guarded_f32((B, H, M)) if guard else empty_f32((B, H, M))
    lib.fa_fwd(wl.dtype, q, k, v, o, lse, B, H, M, N, D, wl.causal, wl.sm_scale)
    out = {"o": o, "lse": lse}
    if with_bwd:
        dq, dk, dv = (alloc(x.shape, wl.dtype) for x in (q, k, v))
        if steps:
            delta = guarded_f32((B, H, M)) if guard else empty_f32((B, H, M))
            lib.fa_bwd_delta(wl.dtype, o, do, dlse, delta, B, H, M, D)
            lib.fa_bwd_dkdv(wl.dtype, q, k, v, do, lse, delta, dk, dv, B, H, M, N, D, wl.causal, wl.sm_scale)
            lib.fa_bwd_dq(wl.dtype, q, k, v, do, lse, delta, dq, B, H, M, N, D, wl.causal, wl.sm_scale)
        else:
            ws_bytes = lib.fa_bwd_workspace_size(B, H, M, N, D, wl.dtype)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
            if dlse is None:
                lib.fa_bwd(wl.dtype, q, k, v, o, do, lse, dq, dk, dv, ws, ws_bytes, B, H, M, N, D,
                           wl.causal, wl.sm_scale)
            else:
                lib.fa_bwd_dlse(wl.dtype, q, k, v, o, do, lse, dlse, dq, dk, dv, ws, ws_bytes, B, H, M, N, D,
                                wl.causal, wl.sm_scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    res = {kk: host(vv) for kk, vv in out.items()}
    if guard:
        check_guards()
    return res


def compare(wl, t, got, heads=None, with_bwd=True, dlse=None):
    sel = (slice(None), slice(None)) if heads is None else None
    c = wl.scale()
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)] if heads is None else heads
    for (b, h) in pairs:
        f = {n: t[n].f64[b:b + 1, h:h + 1] for n in ("q", "k", "v", "do")}
        o, lse = oracle.attn_fwd(f["q"], f["k"], f["v"], wl.causal, c)
        tag = f"{wl.name}[b={b},h={h}]"
        check_output(f"{tag}.o", got["o"][b, h], o[0, 0], wl.dtype)
        check_lse(f"{tag}.lse", got["lse"][b, h], lse[0, 0], wl.dtype)
        if with_bwd:
            g = None if dlse is None else dlse[b:b + 1, h:h + 1]
            dq, dk, dv = oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], wl.causal, c, dlse=g)
            terms = lambda: summand_scales(f, wl.causal, c)
            check_grad(f"{tag}.dq", got["dq"][b, h], dq[0, 0], wl.dtype, zero_scale=lambda: terms()[0])
            check_grad(f"{tag}.dk", got["dk"][b, h], dk[0, 0], wl.dtype, zero_scale=lambda: terms()[1])
            check_grad(f"{tag}.dv", got["dv"][b, h], dv[0, 0], wl.dtype)
    del sel


def summand_scales(f, causal, c):
    """Largest summands of dQ = c (P o dP) K and dK = c (P o dP)^t Q before
    the Delta term cancels them (used only when a reference gradient is all
    zeros); a tolerance scale, not a second reference."""
    q, k, v, do = (f[n][0, 0] for n in ("q", "k", "v", "do"))
    M, N = q.shape[0], k.shape[0]
    s = c * q @ k.T
    if causal:
        s = np.where(np.arange(N)[None, :] > np.arange(M)[:, None] + (N - M), -np.inf, s)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(np.where(np.isfinite(mx), s - mx, -np.inf))
    den = e.sum(axis=1, keepdims=True)
    pm = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)
    t = np.abs(pm * (do @ v.T))
    return c * (t @ np.abs(k)).max(), c * (t.T @ np.abs(q)).max()


SMALL = [
    # dtype, B, H, M, N, D, causal
    (BF16, 2, 3, 192, 192, 128, True),
    (BF16, 2, 3, 192, 192, 128, False),
    (F16, 1, 2, 256, 256, 64, True),
    (F16, 1, 2, 256, 256, 64, False),
    (BF16, 1, 2, 64, 64, 64, True),
    (BF16, 1, 2, 128, 320, 128, True),    # M < N: rows see a longer prefix
    (F16, 1, 2, 320, 128, 64, True),      # M > N: the first 192 rows see no key
    (F16, 1, 2, 128, 320, 128, False),
    (F32, 1, 2, 128, 128, 64, False),
    (F32, 1, 2, 192, 128, 128, True),
    (F32, 1, 1, 64, 192, 64, True),
    # lengths that are not tile multiples: partial last query / key tiles
    (BF16, 2, 3, 200, 200, 128, True),
    (BF16, 2, 3, 200, 200, 128, False),
    (F16, 1, 2, 77, 150, 64, True),       # M < N, both ragged
    (F16, 1, 2, 150, 77, 64, False),      # M > N
    (F16, 1, 2, 150, 77, 128, True),      # M > N causal: rows that see no key
    (BF16, 1, 2, 37, 29, 128, True),      # both below one tile
    (BF16, 1, 2, 29, 37, 64, False),
    (F16, 1, 1, 1, 1, 64, False),         # a single score
    (BF16, 1, 2, 300, 1000, 128, True),   # causal key tail past a full tile
    (BF16, 1, 1, 64, 65, 128, False),     # one key past a tile
    (F32, 1, 2, 100, 130, 64, True),
    # head dims 32 and (fp32) 256
    (BF16, 1, 2, 200, 150, 32, True),
    (F16, 2, 2, 128, 128, 32, False),
    (F16, 1, 2, 77, 300, 32, True),
    (F32, 1, 2, 100, 77, 32, True),
    (F32, 1, 1, 64, 96, 256, True),
    (F32, 1, 1, 70, 50, 256, False),
    # head dim 16 (16-bit: the D = 32 kernels over zero-padded rows; fp32:
    # the generic kernels) and 16-bit 256
    (BF16, 1, 2, 100, 130, 16, True),
    (F16, 2, 1, 64, 64, 16, False),
    (F32, 1, 2, 77, 50, 16, True),
    (BF16, 2, 3, 512, 384, 16, True),     # several blocks, M > N: rows that see no key
    (F16, 1, 2, 200, 1000, 16, False),    # M < N, ragged, partial key block first
    (BF16, 1, 1, 1, 1, 16, True),         # a single score
    (BF16, 1, 2, 130, 100, 256, True),
    (F16, 1, 1, 64, 96, 256, False),
]


@pytest.mark.parametrize("case", [(BF16, 2, 2, 200, 300, 256, True), (F16, 1, 2, 256, 256, 256, False),
                                  (BF16, 1, 2, 128, 128, 256, True), (F16, 1, 1, 33, 65, 256, False),
                                  (BF16, 1, 2, 512, 512, 256, True), (F16, 1, 2, 300, 150, 256, True),
                                  (BF16, 1, 1, 384, 640, 256, False)],
                         ids=lambda c: "-".join(map(str, c)))
def test_head_dim_256(case):
    """fp16/bf16 D = 256 forward and backward on the MFMA kernels (the
    backward passes run one wave per SIMD with two-stage rings): several
    query and key blocks, ragged lengths, M > N causal rows that see no
    key."""
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("d256", dtype, B, H, M, N, D, causal, seed=13 + M + N)
    log(f"fa d256 forward + backward parity {case}")
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t, guard=True)
    compare(wl, t, got)


def test_head_dim_256_steps():
    """D = 256 through the separate Delta, dK/dV and dQ entry points."""
    wl = AttnWorkload("d256_steps", BF16, 1, 2, 256, 320, 256, True, seed=17)
    log("fa d256 backward steps parity")
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t, steps=True, guard=True)
    compare(wl, t, got)


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_small_parity(case):
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("small", dtype, B, H, M, N, D, causal, seed=11 + M + N + D)
    log(f"fa small parity {case}")
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t, guard=True)
    compare(wl, t, got)


LSE_GRAD = [
    (BF16, 1, 2, 256, 256, 128, True),
    (F16, 1, 2, 150, 77, 64, True),       # rows that see no key get a gradient too
    (BF16, 1, 2, 200, 130, 64, False),
    (F32, 1, 2, 128, 192, 64, False),
]


@pytest.mark.parametrize("steps", [False, True], ids=["fused", "steps"])
@pytest.mark.parametrize("case", LSE_GRAD, ids=lambda c: "-".join(map(str, c)))
def test_lse_gradient(case, steps):
    """A gradient reaching LSE (dlse) on top of dO, through fa_bwd and through
    its three steps."""
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("dlse", dtype, B, H, M, N, D, causal, seed=21 + M + N)
    log(f"fa lse-gradient parity {case} steps={steps}")
    t = attn_inputs(wl)
    g = draw(wl.seed + 1, [("dlse", (B, H, M), 1.0, F32)])["dlse"]
    got = run_fwd_bwd(wl, t, steps=steps, guard=True, dlse=dev(g))
    compare(wl, t, got, dlse=g.f64)


def test_steps_equal_fused_bwd():
    """fa_bwd == fa_bwd_delta + fa_bwd_dkdv + fa_bwd_dq, bit for bit."""
    wl = AttnWorkload("steps", BF16, 1, 2, 256, 256, 128, True, seed=5)
    t = attn_inputs(wl)
    a = run_fwd_bwd(wl, t, steps=False)
    b = run_fwd_bwd(wl, t, steps=True)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("case", [(BF16, 1, 2, 256, 256, 128, True, False), (F16, 2, 2, 300, 200, 64, False, True),
                                  (BF16, 1, 3, 130, 250, 32, True, True), (F16, 1, 2, 512, 512, 128, False, False),
                                  (F32, 1, 2, 128, 192, 64, True, True)],
                         ids=lambda c: "-".join(map(str, c)))
def test_dq_delta_equals_steps(case):
    """fa_bwd_dq_delta forms the same Delta as fa_bwd_delta (bit for bit,
    with and without an LSE gradient) and the same dq as fa_bwd_dq reading it."""
    torch = need_gpu()
    dtype, B, H, M, N, D, causal, with_dlse = case
    wl = AttnWorkload("dq_delta", dtype, B, H, M, N, D, causal, seed=9 + M)
    log(f"dq+delta vs steps {case}")
    t = attn_inputs(wl)
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    dlse = dev(draw(wl.seed + 1, [("dlse", (B, H, M), 1.0, F32)])["dlse"]) if with_dlse else None
    o, lse = filled((B, H, M, D), dtype), empty_f32((B, H, M))
    lib.fa_fwd(dtype, q, k, v, o, lse, B, H, M, N, D, causal, wl.sm_scale)
    d1, d2 = guarded_f32((B, H, M)), guarded_f32((B, H, M))
    q1, q2 = guarded((B, H, M, D), dtype), guarded((B, H, M, D), dtype)
    lib.fa_bwd_delta(dtype, o, do, dlse, d1, B, H, M, D)
    lib.fa_bwd_dq(dtype, q, k, v, do, lse, d1, q1, B, H, M, N, D, causal, wl.sm_scale)
    lib.fa_bwd_dq_delta(dtype, q, k, v, o, do, lse, dlse, d2, q2, B, H, M, N, D, causal, wl.sm_scale)
    torch.cuda.synchronize()
    check_guards()
    assert np.array_equal(host(d1), host(d2)), "delta"
    assert np.array_equal(host(q1), host(q2)), "dq"


DET_CASES = [
    # dtype, B, H, M, N, D, causal: one case per kernel family
    (F16, 1, 4, 256, 256, 64, False),     # pipelined forward at D = 64
    (BF16, 1, 4, 1024, 1024, 128, True),  # the pipelined causal D = 128 forward and its passes, several workgroups
    (BF16, 1, 2, 576, 512, 256, True),    # head dim 256 (one wave per SIMD), M > N
    (BF16, 1, 2, 333, 517, 16, False),    # head dim 16 (zero-padded D = 32 tiles), ragged
    (F32, 1, 2, 200, 170, 64, True),      # the generic fp32 kernels
]


@pytest.mark.parametrize("case", DET_CASES, ids=lambda c: "-".join(map(str, c)))
def test_deterministic(case):
    """No float atomics anywhere: two runs on the same inputs give bitwise-equal outputs."""
    dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("det", dtype, B, H, M, N, D, causal, seed=6 + M + D)
    log(f"determinism {case}")
    t = attn_inputs(wl)
    a = run_fwd_bwd(wl, t)
    b = run_fwd_bwd(wl, t)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_noncausal_bwd_sees_all_queries():
    """A backward that walks only the causal band (the defect discussed in the
    tutorial's comment thread) would give the same dK for causal and
    non-causal inputs on the first key block; the oracle says they differ and
    the kernel must follow the oracle."""
    wl = AttnWorkload("nc", BF16, 1, 2, 256, 256, 64, False, seed=8)
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t)
    compare(wl, t, got)
    wlc = AttnWorkload("c", BF16, 1, 2, 256, 256, 64, True, seed=8)
    gotc = run_fwd_bwd(wlc, t)
    assert np.abs(got["dk"][:, :, :64] - gotc["dk"][:, :, :64]).max() > 0.1


@pytest.mark.parametrize("D", [128, 256, 16, 32])
def test_large_scale_peaky_softmax(D):
    """sm_scale 1.0 makes rows nearly one-hot (large logits, many lazy
    rescales), on each head-dim path: the pipelined D = 128 forward, the
    one-wave-per-SIMD D = 256 passes, the D = 32 kernels and D = 16 over
    zero-padded rows."""
    wl = AttnWorkload("peaky", BF16, 1, 2, 256, 256, D, True, seed=9, sm_scale=1.0)
    log(f"peaky softmax D = {D}")
    t = attn_inputs(wl)
    compare(wl, t, run_fwd_bwd(wl, t))


MANY_WG = [
    # dtype, B, H, M, N, D, causal, heads checked (None: all)
    (BF16, 8, 16, 1024, 1024, 128, True, [(0, 0), (3, 7), (7, 15)]),   # 512 workgroups: two rounds per CU
    (F16, 1, 24, 2816, 512, 64, False, [(0, 0), (0, 13), (0, 23)]),    # heads not a multiple of 8
    (BF16, 1, 3, 256, 768, 128, True, None),                            # causal with M < N
    (F16, 2, 5, 512, 512, 64, True, None),
]


@pytest.mark.parametrize("case", MANY_WG, ids=lambda c: "-".join(map(str, c[:7])))
def test_forward_workgroup_schedules(case):
    """More workgroups than CUs, head counts that are and are not multiples
    of 8, causal with M < N: every output finite, the listed heads against
    the oracle."""
    dtype, B, H, M, N, D, causal, heads = case
    wl = AttnWorkload("sched", dtype, B, H, M, N, D, causal, seed=71 + M + H)
    log(f"forward schedule {case[:7]}")
    t = attn_inputs(wl, ("q", "k", "v", "do"))
    got = run_fwd_bwd(wl, t, with_bwd=False, guard=True)
    assert np.all(np.isfinite(got["o"])) and np.all(np.isfinite(got["lse"]))
    compare(wl, t, got, heads=heads, with_bwd=False)


_FULL = {}


def full_size_run(name):
    """GPU outputs (host fp64) and inputs of a full-size workload, computed
    once per test session: the per-head oracle comparisons below are split
    into chunks so that each test stays short."""
    if name not in _FULL:
        wl = WORKLOADS[name]
        log(f"fa full-size {name}: GPU run")
        t = attn_inputs(wl)
        _FULL.clear()
        _FULL[name] = (wl, t, run_fwd_bwd(wl, t))
    return _FULL[name]


FULL_CHUNKS = 4


@pytest.mark.parametrize("chunk", range(FULL_CHUNKS))
def test_full_size_causal_all_heads(chunk):
    """Causal bf16 B4 H16 2048 D128, every head against the oracle (O, LSE,
    dQ, dK, dV), in four chunks of 16 heads."""
    wl, t, got = full_size_run("causal_bf16_b4h16_s2048_d128")
    pairs = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    per = len(pairs) // FULL_CHUNKS
    heads = pairs[chunk * per:(chunk + 1) * per]
    log(f"fa full-size causal heads {heads[0]}..{heads[-1]}")
    compare(wl, t, got, heads=heads)


def test_full_size_noncausal_sampled_heads():
    """Non-causal bf16 B1 H32 8192 D128: the first, a middle and the last
    head against the oracle; every output of every head finite (the buffers
    start as NaN, so an element no kernel wrote fails)."""
    wl, t, got = full_size_run("noncausal_bf16_b1h32_s8192_d128")
    for n, x in got.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values"
    compare(wl, t, got, heads=[(0, 0), (0, 17), (0, 31)])
    _FULL.clear()


@pytest.mark.parametrize("D", [256, 16])
def test_head_dims_bench_shape_sampled_heads(D):
    """The head-dim workloads the benchmark times (causal bf16 B1 H16
    2048^2, D = 256 on the matrix cores, D = 16 on the generic kernels):
    every output finite, three heads against the oracle (O, LSE, dQ, dK,
    dV)."""
    wl = AttnWorkload(f"causal_bf16_b1h16_s2048_d{D}", BF16, 1, 16, 2048, 2048, D, True, seed=6)
    log(f"fa head-dim bench shape D = {D}")
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values"
    compare(wl, t, got, heads=[(0, 0), (0, 7), (0, 15)])


def test_full_size_tiny_f32():
    """The tiny fp32 workload (B1 H2 128x128 D64, non-causal) against the
    literal fp32 bar: max-abs error <= 1e-4 on O, LSE, dQ, dK and dV."""
    wl = WORKLOADS["tiny_f32"]
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t)
    f = {n: t[n].f64 for n in ("q", "k", "v", "do")}
    o, lse = oracle.attn_fwd(f["q"], f["k"], f["v"], wl.causal, wl.scale())
    dq, dk, dv = oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], wl.causal, wl.scale())
    for n, ref in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        err = check_fp32_abs(f"tiny_f32.{n}", got[n], ref)
        log(f"tiny_f32.{n}: max abs err {err:.2e}")
