"""GPU parity: resmerge_fwd / resmerge_bwd and lse_merge_fwd / lse_merge_bwd
against the fp64 oracle."""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16, F16, F32, MERGE_WORKLOAD, MergeWorkload, draw, merge_inputs
from gpu_util import check_guards, dev, empty, empty_f32, filled, guarded, guarded_f32, host, log, need_gpu
from tolerance import check_grad, check_lse, check_output

pytestmark = pytest.mark.gpu


def run_merge(wl, t, with_gl=True, l0=None):
    torch = need_gpu()
    x, y0, q, gy = (dev(t[n]) for n in ("x", "y0", "q", "gy"))
    l0d = dev(t["l0"]) if l0 is None else torch.from_numpy(l0.astype(np.float32)).cuda()
    gl = dev(t["gl"]) if with_gl else None
    R, D = wl.rows, wl.D
    y = guarded((R, D), wl.dtype)
    lse = guarded_f32((R,))
    lib.resmerge_fwd(wl.dtype, x, q, y0, l0d, y, lse, R, D, wl.eps)
    gx, gy0 = guarded((R, D), wl.dtype), guarded((R, D), wl.dtype)
    gq, gl0 = guarded_f32((D,)), guarded_f32((R,))
    nb = lib.resmerge_bwd_workspace_size(R, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lib.resmerge_bwd(wl.dtype, x, q, y0, l0d, gy, gl, gx, gq, gy0, gl0, ws, nb, R, D, wl.eps)
    torch.cuda.synchronize()
    res = {n: host(v) for n, v in (("y", y), ("lse", lse), ("gx", gx), ("gq", gq), ("gy0", gy0),
                                   ("gl0", gl0))}
    check_guards()
    return res


def compare(wl, t, got, with_gl=True, l0=None):
    f = {n: t[n].f64 for n in ("x", "q", "y0", "l0", "gy", "gl")}
    if l0 is not None:
        f["l0"] = l0
    y, lse = oracle.merge_fwd(f["x"], f["q"], f["y0"], f["l0"], wl.eps)
    gx, gq, gy0, gl0 = oracle.merge_bwd(f["x"], f["q"], f["y0"], f["l0"], f["gy"],
                                        f["gl"] if with_gl else None, wl.eps)
    tag = wl.name
    check_output(f"{tag}.y", got["y"], y, wl.dtype)
    check_lse(f"{tag}.lse", got["lse"], lse, wl.dtype)
    check_grad(f"{tag}.gx", got["gx"], gx, wl.dtype)
    check_grad(f"{tag}.gq", got["gq"], gq, wl.dtype)
    check_grad(f"{tag}.gy0", got["gy0"], gy0, wl.dtype)
    check_grad(f"{tag}.gl0", got["gl0"], gl0, wl.dtype)


SMALL = [
    # dtype, rows, D, eps          register path: 16-byte chunks per row C = 64 * WPR * NCH
    (BF16, 37, 4096, 1e-6),       # WPR 4, NCH 2, ragged row count
    (F16, 300, 1024, 1e-6),       # WPR 1 (one wavefront per row), NCH 2
    (BF16, 129, 512, 1.1920929e-07),  # WPR 1, NCH 1
    (F32, 50, 2048, 1e-6),        # WPR 4, NCH 2 (4 elements per chunk)
    (F32, 17, 8192, 1e-6),        # WPR 4, NCH 8
    (BF16, 1000, 2048, 1e-6),     # WPR 4, NCH 1
    (BF16, 77, 8192, 1e-6),       # WPR 4, NCH 4
    (F16, 50, 16384, 1e-6),       # WPR 4, NCH 8
    (BF16, 33, 1000, 1e-6),       # generic path (D not a whole number of chunks per thread)
    (F16, 5000, 24, 1e-6),        # generic path, tiny rows, many of them
    (BF16, 9000, 3072, 1e-6),     # generic path, more rows than wavefronts
    (BF16, 3000, 4096, 1e-6),     # more rows than resident workgroups: grid-stride loop
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "-".join(map(str, c)))
def test_merge_small(case):
    dtype, rows, D, eps = case
    wl = MergeWorkload("merge_small", dtype, rows, D, eps, seed=40 + rows)
    log(f"merge small parity {case}")
    t = merge_inputs(wl)
    compare(wl, t, run_merge(wl, t))


def test_merge_without_gl_and_with_neg_inf_l0():
    wl = MergeWorkload("merge_edge", BF16, 64, 4096, 1e-6, seed=44)
    t = merge_inputs(wl)
    l0 = t["l0"].f64.copy()
    l0[::3] = -np.inf
    got = run_merge(wl, t, with_gl=False, l0=l0)
    compare(wl, t, got, with_gl=False, l0=l0)
    # l0 = -inf rows return x exactly (alpha = 0, beta = 1)
    np.testing.assert_array_equal(got["y"][::3], t["x"].f64[::3])
    assert np.all(got["gy0"][::3] == 0) and np.all(got["gl0"][::3] == 0)


def test_merge_deterministic():
    wl = MergeWorkload("merge_det", BF16, 2048, 4096, 1e-6, seed=45)
    t = merge_inputs(wl)
    a = run_merge(wl, t)
    b = run_merge(wl, t)
    for n in a:
        assert np.array_equal(a[n], b[n]), n


def test_merge_full_size():
    wl = MERGE_WORKLOAD
    log("merge full-size")
    t = merge_inputs(wl)
    compare(wl, t, run_merge(wl, t))


@pytest.mark.parametrize("case", [(BF16, 37, 4096, 1e-6), (F32, 50, 2048, 1e-6), (BF16, 33, 1000, 1e-6),
                                  (F16, 300, 1024, 1e-6)], ids=lambda c: "-".join(map(str, c)))
def test_merge_bwd_accumulate(case):
    """accumulate = 1 adds gx and gq into what the buffers hold (the page's
    atomic-add semantics); gy0 and gl0 are overwritten as in mode 0."""
    torch = need_gpu()
    dtype, R, D, eps = case
    wl = MergeWorkload("merge_acc", dtype, R, D, eps, seed=81 + D)
    log(f"merge accumulate {case}")
    t = merge_inputs(wl)
    prior = draw(wl.seed + 1, [("gx0", (R, D), 1.0, dtype), ("gq0", (D,), 1.0, F32)])
    x, y0, q, gy, l0, gl = (dev(t[n]) for n in ("x", "y0", "q", "gy", "l0", "gl"))
    gx, gy0 = guarded((R, D), dtype), guarded((R, D), dtype)
    gq, gl0 = guarded_f32((D,)), guarded_f32((R,))
    gx.copy_(dev(prior["gx0"]))
    gq.copy_(dev(prior["gq0"]))
    nb = lib.resmerge_bwd_workspace_size(R, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    lib.resmerge_bwd_acc(dtype, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, ws, nb, R, D, eps, 1)
    torch.cuda.synchronize()
    got = {n: host(v) for n, v in (("gx", gx), ("gq", gq), ("gy0", gy0), ("gl0", gl0))}
    check_guards()
    f = {n: t[n].f64 for n in ("x", "q", "y0", "l0", "gy", "gl")}
    rgx, rgq, rgy0, rgl0 = oracle.merge_bwd(f["x"], f["q"], f["y0"], f["l0"], f["gy"], f["gl"], eps)
    tag = f"merge_acc{case}"
    check_grad(tag + ".gx", got["gx"], prior["gx0"].f64 + rgx, dtype)
    check_grad(tag + ".gq", got["gq"], prior["gq0"].f64 + rgq, dtype)
    check_grad(tag + ".gy0", got["gy0"], rgy0, dtype)
    check_grad(tag + ".gl0", got["gl0"], rgl0, dtype)


# ------------------------------------------------------ N-way lse merge ----

LSE_MERGE = [
    # dtype, S, rows, D     lanes per row x chunks per lane
    (BF16, 4, 1000, 128),   # 16 x 1
    (F16, 1, 77, 64),       # 8 x 1, a single input
    (F32, 3, 50, 40),       # 8 x 1 with 3 idle lanes per row
    (BF16, 2, 300, 4096),   # 64 x 8
    (BF16, 5, 129, 1000),   # 64 x 2, partial last chunk round
    (F16, 8, 333, 8),       # 1 x 1
    (BF16, 12, 200, 128),   # 16 x 1 with more than 8 inputs (the path that reads them twice)
    (F32, 7, 90, 512),      # 64 x 1, the widest rows kept in registers
]


def _lm_inputs(dtype, S, rows, D, seed, neg_inf=True):
    t = draw(seed, [("ys", (S, rows, D), 1.0, dtype), ("lses", (S, rows), 2.0, F32),
                    ("gy", (rows, D), 1.0, dtype), ("gl", (rows,), 1.0, F32)])
    lses = t["lses"].f64.copy()
    if neg_inf and S > 1:
        lses[1, ::7] = -np.inf          # an input that contributes nothing to some rows
        lses[:, 3 % rows] = -np.inf     # a row that sees nothing at all
    return t, lses


@pytest.mark.parametrize("case", LSE_MERGE, ids=lambda c: "-".join(map(str, c)))
@pytest.mark.parametrize("with_gl", [True, False], ids=["gl", "no_gl"])
def test_lse_merge_parity(case, with_gl):
    torch = need_gpu()
    dtype, S, rows, D = case
    log(f"lse_merge parity {case} gl={with_gl}")
    t, lses = _lm_inputs(dtype, S, rows, D, seed=91 + S + D)
    ys, gy = dev(t["ys"]), dev(t["gy"])
    ls = torch.from_numpy(lses.astype(np.float32)).cuda()
    gl = dev(t["gl"]) if with_gl else None
    y, lse = guarded((rows, D), dtype), guarded_f32((rows,))
    gys, gls = guarded((S, rows, D), dtype), guarded_f32((S, rows))
    lib.lse_merge_fwd(dtype, ys, ls, y, lse, S, rows, D)
    lib.lse_merge_bwd(dtype, ys, ls, gy, gl, gys, gls, S, rows, D)
    torch.cuda.synchronize()
    got = {n: host(v) for n, v in (("y", y), ("lse", lse), ("gys", gys), ("gls", gls))}
    check_guards()
    ry, rl = oracle.lse_merge_fwd(t["ys"].f64, lses)
    rgy, rgl = oracle.lse_merge_bwd(t["ys"].f64, lses, t["gy"].f64, t["gl"].f64 if with_gl else None)
    tag = f"lse_merge{case}"
    check_output(tag + ".y", got["y"], ry, dtype)
    check_lse(tag + ".lse", got["lse"], rl, dtype)
    check_grad(tag + ".gys", got["gys"], rgy, dtype)
    check_grad(tag + ".glses", got["gls"], rgl, dtype)
    if S > 1:
        dead = np.isneginf(lses)
        assert np.all(got["gys"][dead] == 0) and np.all(got["gls"][dead] == 0)


def test_split_keys_attention_merge():
    """Split-KV attention: fa_fwd on three ragged key ranges, merged by
    lse_merge_fwd, against the oracle's attention over all keys."""
    torch = need_gpu()
    from attention_fa2_tiles_amd.inputs import AttnWorkload, attn_inputs
    B, H, M, D = 1, 4, 200, 128
    splits = [100, 77, 123]
    N = sum(splits)
    wl = AttnWorkload("split", BF16, B, H, M, N, D, False, seed=97)
    t = attn_inputs(wl, ("q", "k", "v"))
    q, k, v = (dev(t[n]) for n in ("q", "k", "v"))
    S, rows = len(splits), B * H * M
    ys = torch.empty((S, B, H, M, D), dtype=torch.bfloat16, device="cuda")
    ls = torch.empty((S, B, H, M), dtype=torch.float32, device="cuda")
    j = 0
    for s, n in enumerate(splits):
        ks, vs = k[:, :, j:j + n].contiguous(), v[:, :, j:j + n].contiguous()
        lib.fa_fwd(BF16, q, ks, vs, ys[s], ls[s], B, H, M, n, D, 0, 0.0)
        j += n
    y, lse = guarded((rows, D), BF16), guarded_f32((rows,))
    lib.lse_merge_fwd(BF16, ys, ls, y, lse, S, rows, D)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(t["q"].f64, t["k"].f64, t["v"].f64, False, wl.scale())
    check_output("split.o", host(y), ro.reshape(rows, D), BF16)
    check_lse("split.lse", host(lse), rl.reshape(rows), BF16)
    check_guards()
