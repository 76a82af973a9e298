"""GPU parity at tensor sizes past 2^31 elements.

Every kernel forms its element offsets in 64-bit arithmetic (head or row
index times the row length); a 32-bit product would wrap for the heads or
rows whose offsets pass 2^31.  These tests run the production kernels on
tensors just past that size (4 GiB of bf16 each) and compare the heads or
rows on both sides of the 2^31 boundary, and the first and last ones, with
the fp64 oracle.

Inputs: N(0, 1) (the merge's pseudo-query N(0, 1/D)) drawn on the device by
torch's seeded generator straight into bf16 tensors -- drawing 4 GiB
tensors on the host would dominate the run -- and the sampled heads or rows
are read back as the oracle's inputs.
"""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16
from gpu_util import host, log, need_gpu
from tolerance import check_grad, check_lse, check_output

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31


def _normal(torch, gen, shape, std=1.0, dtype=None):
    x = torch.empty(shape, dtype=dtype or torch.bfloat16, device="cuda")
    x.normal_(0.0, std, generator=gen)
    return x


def _release(torch):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_attention_offsets_past_2_31(causal):
    """bf16 B4 H32770 M=N=128 D128 (2^31 + 2^17 elements per tensor):
    fa_fwd then fa_bwd; heads 0, the two around the 2^31 element offset and
    the last head against the oracle (O, LSE, dQ, dK, dV)."""
    torch = need_gpu()
    B, H, M, N, D = 4, 32770, 128, 128, 128
    assert B * H * M * D > TWO31
    scale = 1.0 / np.sqrt(D)
    gen = torch.Generator(device="cuda").manual_seed(71 + int(causal))
    log(f"attention past 2^31 elements, causal={causal}: drawing inputs")
    q, k, v, do = (_normal(torch, gen, (B, H, M, D)) for _ in range(4))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    lse = torch.empty((B, H, M), dtype=torch.float32, device="cuda")
    nb = lib.fa_bwd_workspace_size(B, H, M, N, D, BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    log("fa_fwd + fa_bwd")
    lib.fa_fwd(BF16, q, k, v, o, lse, B, H, M, N, D, causal, scale)
    lib.fa_bwd(BF16, q, k, v, o, do, lse, dq, dk, dv, ws, nb, B, H, M, N, D, causal, scale)
    torch.cuda.synchronize()
    first_past = TWO31 // (M * D)           # the first head whose offset is >= 2^31
    flat_heads = [0, first_past - 1, first_past, B * H - 1]
    for bh in flat_heads:
        b, h = divmod(bh, H)
        f = {n: host(t[b:b + 1, h:h + 1]) for n, t in (("q", q), ("k", k), ("v", v), ("do", do))}
        ro, rl = oracle.attn_fwd(f["q"], f["k"], f["v"], causal, scale)
        rdq, rdk, rdv = oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], causal, scale)
        tag = f"large[{b},{h}]"
        check_output(tag + ".o", host(o[b:b + 1, h:h + 1]), ro, BF16)
        check_lse(tag + ".lse", host(lse[b:b + 1, h:h + 1]), rl, BF16)
        check_grad(tag + ".dq", host(dq[b:b + 1, h:h + 1]), rdq, BF16)
        check_grad(tag + ".dk", host(dk[b:b + 1, h:h + 1]), rdk, BF16)
        check_grad(tag + ".dv", host(dv[b:b + 1, h:h + 1]), rdv, BF16)
        log(f"{tag} (flat head {bh}, element offset {bh * M * D}) ok")
    del q, k, v, do, o, dq, dk, dv, lse, ws
    _release(torch)


def test_residual_merge_offsets_past_2_31():
    """bf16 rows = 2^19 + 2, D = 4096 (2^31 + 8192 elements per row tensor):
    resmerge_fwd and resmerge_bwd; rows 0, the two around the 2^31 element
    offset and the last row against the oracle (y, lse, gx, gy0, gl0; gq is
    a sum over every row and is covered at smaller sizes)."""
    torch = need_gpu()
    R, D, eps = (1 << 19) + 2, 4096, 1e-6
    assert R * D > TWO31
    gen = torch.Generator(device="cuda").manual_seed(73)
    log("residual merge past 2^31 elements: drawing inputs")
    x, y0, gy = (_normal(torch, gen, (R, D)) for _ in range(3))
    q = _normal(torch, gen, (D,), std=1.0 / np.sqrt(D))
    l0 = _normal(torch, gen, (R,), dtype=torch.float32)
    gl = _normal(torch, gen, (R,), dtype=torch.float32)
    y, gx, gy0 = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    lse, gl0 = torch.empty(R, dtype=torch.float32, device="cuda"), torch.empty(R, dtype=torch.float32, device="cuda")
    gq = torch.empty(D, dtype=torch.float32, device="cuda")
    nb = lib.resmerge_bwd_workspace_size(R, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    log("resmerge_fwd + resmerge_bwd")
    lib.resmerge_fwd(BF16, x, q, y0, l0, y, lse, R, D, eps)
    lib.resmerge_bwd(BF16, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, ws, nb, R, D, eps)
    torch.cuda.synchronize()
    first_past = TWO31 // D
    rows = [0, first_past - 1, first_past, R - 1]
    qh = host(q)
    for r in rows:
        f = {n: host(t[r:r + 1]) for n, t in (("x", x), ("y0", y0), ("gy", gy), ("l0", l0), ("gl", gl))}
        ry, rlse = oracle.merge_fwd(f["x"], qh, f["y0"], f["l0"], eps)
        rgx, _, rgy0, rgl0 = oracle.merge_bwd(f["x"], qh, f["y0"], f["l0"], f["gy"], f["gl"], eps)
        tag = f"large_merge[{r}]"
        check_output(tag + ".y", host(y[r:r + 1]), ry, BF16)
        check_lse(tag + ".lse", host(lse[r:r + 1]), rlse, BF16)
        check_grad(tag + ".gx", host(gx[r:r + 1]), rgx, BF16)
        check_grad(tag + ".gy0", host(gy0[r:r + 1]), rgy0, BF16)
        check_grad(tag + ".gl0", host(gl0[r:r + 1]), rgl0, BF16)
        log(f"{tag} (element offset {r * D}) ok")
    assert bool(torch.isfinite(gq).all())
    del x, y0, gy, q, l0, gl, y, gx, gy0, lse, gl0, gq, ws
    _release(torch)


def test_lse_merge_offsets_past_2_31():
    """bf16 S = 4 partials of rows = 2^22 + 2, D = 128 (2^31 + 1024
    elements in ys): lse_merge_fwd and lse_merge_bwd; rows 0, the two around
    the row where the last partial passes offset 2^31, and the last row."""
    torch = need_gpu()
    S, R, D = 4, (1 << 22) + 2, 128
    assert S * R * D > TWO31
    gen = torch.Generator(device="cuda").manual_seed(79)
    log("N-way merge past 2^31 elements: drawing inputs")
    ys = _normal(torch, gen, (S, R, D))
    lses = _normal(torch, gen, (S, R), std=2.0, dtype=torch.float32)
    gy = _normal(torch, gen, (R, D))
    gl = _normal(torch, gen, (R,), dtype=torch.float32)
    y, lse = torch.empty((R, D), dtype=torch.bfloat16, device="cuda"), torch.empty(R, dtype=torch.float32, device="cuda")
    gys, glses = torch.empty_like(ys), torch.empty_like(lses)
    log("lse_merge_fwd + lse_merge_bwd")
    lib.lse_merge_fwd(BF16, ys, lses, y, lse, S, R, D)
    lib.lse_merge_bwd(BF16, ys, lses, gy, gl, gys, glses, S, R, D)
    torch.cuda.synchronize()
    first_past = TWO31 // D - (S - 1) * R    # first row of partial S-1 at offset >= 2^31
    rows = [0, first_past - 1, first_past, R - 1]
    for r in rows:
        f_ys = host(ys[:, r:r + 1])
        f_l = host(lses[:, r:r + 1])
        ry, rl = oracle.lse_merge_fwd(f_ys, f_l)
        rgys, rgl = oracle.lse_merge_bwd(f_ys, f_l, host(gy[r:r + 1]), host(gl[r:r + 1]))
        tag = f"large_lse_merge[{r}]"
        check_output(tag + ".y", host(y[r:r + 1]), ry, BF16)
        check_lse(tag + ".lse", host(lse[r:r + 1]), rl, BF16)
        check_grad(tag + ".gys", host(gys[:, r:r + 1]), rgys, BF16)
        check_grad(tag + ".glses", host(glses[:, r:r + 1]), rgl, BF16)
        log(f"{tag} (last partial's element offset {((S - 1) * R + r) * D}) ok")
    del ys, lses, gy, gl, y, lse, gys, glses
    _release(torch)
