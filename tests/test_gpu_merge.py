"""GPU parity: resmerge_fwd / resmerge_bwd against the fp64 oracle."""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16, F16, F32, MERGE_WORKLOAD, MergeWorkload, merge_inputs
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
