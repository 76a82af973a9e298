"""GPU: fa_bwd_noalloc (the backward whose Delta lives in the library's own
device array, for callers that cannot allocate) gives exactly fa_bwd's
gradients, on two calls in a row, the second on a smaller problem, through
the C ABI.  Bitwise equality is asked: both run the same kernels on the same
inputs, only the buffer that holds Delta differs."""

import numpy as np
import pytest

from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16, F32, AttnWorkload, attn_inputs
from gpu_util import check_guards, dev, empty_f32, guarded, host, log, need_gpu

pytestmark = pytest.mark.gpu


def grads(wl, t, noalloc):
    torch = need_gpu()
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o = guarded((B, H, M, D), wl.dtype)
    lse = empty_f32((B, H, M))
    lib.fa_fwd(wl.dtype, q, k, v, o, lse, B, H, M, N, D, wl.causal, wl.sm_scale)
    dq, dk, dv = (guarded(x.shape, wl.dtype) for x in (q, k, v))
    if noalloc:
        lib.fa_bwd_noalloc(wl.dtype, q, k, v, o, do, lse, dq, dk, dv, B, H, M, N, D, wl.causal, wl.sm_scale)
    else:
        nb = lib.fa_bwd_workspace_size(B, H, M, N, D, wl.dtype)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        lib.fa_bwd(wl.dtype, q, k, v, o, do, lse, dq, dk, dv, ws, nb, B, H, M, N, D, wl.causal, wl.sm_scale)
    torch.cuda.synchronize()
    out = {"dq": host(dq), "dk": host(dk), "dv": host(dv)}
    check_guards()
    return out


# per case: a larger call, then a smaller one (the array keeps the first
# call's rows); head dim 256 runs the one-wave-per-SIMD backward passes
CASES = {
    "bf16": (BF16, [(2, 3, 512, 512, 128, True), (1, 2, 100, 130, 64, False)]),
    "f32": (F32, [(1, 2, 192, 192, 64, True), (1, 1, 70, 50, 32, False)]),
    "bf16_d256": (BF16, [(1, 2, 384, 320, 256, True), (1, 1, 100, 70, 256, False)]),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_backward_matches_fa_bwd(case):
    dtype, shapes = CASES[case]
    for i, (B, H, M, N, D, causal) in enumerate(shapes):
        wl = AttnWorkload("noalloc", dtype, B, H, M, N, D, causal, seed=60 + i)
        log(f"fa_bwd_noalloc vs fa_bwd: dtype {dtype} shape {(B, H, M, N, D, causal)}")
        t = attn_inputs(wl)
        want = grads(wl, t, noalloc=False)
        got = grads(wl, t, noalloc=True)
        for n in ("dq", "dk", "dv"):
            assert np.array_equal(got[n], want[n]), f"{n} differs (shape {i})"
