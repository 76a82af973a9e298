"""Every entry point launches on the stream it is given.

The binding passes torch's current stream when no stream is named, so the
calls below run on a side stream of their own.  That stream is first kept
busy by a device-side sleep, then the outputs are filled with NaN on it, then
the library is called: launched on that stream, its kernels run after the
fill and leave the same results as a run on the default stream (the kernels
are deterministic, so bitwise); launched on any other stream they would run
during the sleep and the fill would leave NaN behind.  (PyTorch's side
streams do not synchronise with the legacy default stream.)
"""

import numpy as np
import pytest

from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import (BF16, F16, F8E5M2, AttnWorkload, LseMergeWorkload, MergeWorkload,
                                            attn_inputs, lse_merge_inputs, merge_inputs)
from gpu_util import dev, empty_f32, filled, host, log, need_gpu

pytestmark = pytest.mark.gpu

SLEEP_CYCLES = 40_000_000  # ~20 ms of one wave spinning at the shader clock


def _calls(torch, seed=0):
    """(outputs, launch) per entry point: launch() enqueues the call on the
    current stream and writes the outputs."""
    out = []
    wl = AttnWorkload("stream_attn", BF16, 1, 2, 384, 320, 128, True, seed=81 + seed)
    t = attn_inputs(wl)
    q, k, v, do = (dev(t[n]) for n in ("q", "k", "v", "do"))
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o, lse = filled((B, H, M, D), BF16), empty_f32((B, H, M))
    dq, dk, dv = filled(q.shape, BF16), filled(k.shape, BF16), filled(v.shape, BF16)
    nb = lib.fa_bwd_workspace_size(B, H, M, N, D, BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")

    def attn():
        lib.fa_fwd(BF16, q, k, v, o, lse, B, H, M, N, D, 1, 0.0)
        lib.fa_bwd(BF16, q, k, v, o, do, lse, dq, dk, dv, ws, nb, B, H, M, N, D, 1, 0.0)
    out.append(("fa_fwd + fa_bwd", [o, lse, dq, dk, dv], attn))

    nq, nk, nv = filled(q.shape, BF16), filled(k.shape, BF16), filled(v.shape, BF16)
    out.append(("fa_bwd_noalloc", [nq, nk, nv],
                lambda: lib.fa_bwd_noalloc(BF16, q, k, v, o, do, lse, nq, nk, nv, B, H, M, N, D, 1, 0.0)))

    wp = AttnWorkload("stream_pw", F16, 1, 2, 256, 256, 64, True, seed=85 + seed)
    pn = ("q1", "k1", "q2", "k2", "v", "do")
    tp = attn_inputs(wp, pn)
    dp = [dev(tp[n]) for n in pn]
    po, pl = filled((1, 2, 256, 64), F16), empty_f32((1, 2, 256))
    pg = [filled((1, 2, 256, 64), F16) for _ in range(5)]
    pnb = lib.pw_bwd_workspace_size(1, 2, 256, 256, 64, F16)
    pws = torch.empty(pnb, dtype=torch.uint8, device="cuda")

    def pw():
        lib.pw_fwd(F16, *dp[:5], po, pl, 1, 2, 256, 256, 64, 1, 0.0, 40)
        lib.pw_bwd(F16, *dp[:5], po, dp[5], pl, *pg, pws, pnb, 1, 2, 256, 256, 64, 1, 0.0, 40)
    out.append(("pw_fwd + pw_bwd", [po, pl] + pg, pw))

    wf = AttnWorkload("stream_fp8", F8E5M2, 1, 2, 256, 256, 128, True, seed=86 + seed)
    tf = attn_inputs(wf, ("q", "k", "v"))
    fq, fk = (torch.from_numpy(tf[n].storage).cuda() for n in ("q", "k"))
    fvt = torch.from_numpy(np.ascontiguousarray(np.swapaxes(tf["v"].storage, 2, 3))).cuda()
    fo, fl = filled((1, 2, 256, 128), BF16), empty_f32((1, 2, 256))
    out.append(("fa_fwd_fp8", [fo, fl],
                lambda: lib.fa_fwd_fp8(BF16, fq, fk, fvt, fo, fl, 1, 2, 256, 256, 128, 1, 0.0)))

    wj = AttnWorkload("stream_jvp", F16, 1, 2, 256, 256, 64, True, seed=82 + seed)
    names = ("q", "k", "v", "tq", "tk", "tv")
    tj = attn_inputs(wj, names)
    dj = [dev(tj[n]) for n in names]
    jo, jto, jl = filled((1, 2, 256, 64), F16), filled((1, 2, 256, 64), F16), empty_f32((1, 2, 256))
    out.append(("fa_fwd_jvp", [jo, jl, jto],
                lambda: lib.fa_fwd_jvp(F16, *dj, jo, jl, jto, 1, 2, 256, 256, 64, 1, 0.0)))

    mw = MergeWorkload("stream_merge", BF16, 96, 1024, 1e-6, 83 + seed)
    tm = merge_inputs(mw)
    x, y0, mq, l0 = (dev(tm[n]) for n in ("x", "y0", "q", "l0"))
    y, mlse = filled((mw.rows, mw.D), BF16), empty_f32((mw.rows,))
    out.append(("resmerge_fwd", [y, mlse],
                lambda: lib.resmerge_fwd(BF16, x, mq, y0, l0, y, mlse, mw.rows, mw.D, mw.eps)))

    lw = LseMergeWorkload("stream_lse_merge", BF16, 3, 200, 128, 84 + seed)
    tl = lse_merge_inputs(lw)
    ys, lses = dev(tl["ys"]), dev(tl["lses"])
    ly, llse = filled((lw.rows, lw.D), BF16), empty_f32((lw.rows,))
    out.append(("lse_merge_fwd", [ly, llse],
                lambda: lib.lse_merge_fwd(BF16, ys, lses, ly, llse, lw.S, lw.rows, lw.D)))
    return out


def test_launches_follow_the_current_stream():
    torch = need_gpu()
    calls = _calls(torch)
    # reference: every call on the default stream
    for _, outs, launch in calls:
        launch()
    torch.cuda.synchronize()
    ref = [[host(x).copy() for x in outs] for _, outs, _ in calls]
    side = torch.cuda.Stream()
    for (name, outs, launch), r in zip(calls, ref):
        log(f"stream order: {name}")
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            torch.cuda._sleep(SLEEP_CYCLES)
            for x in outs:
                x.fill_(float("nan"))
            launch()
        side.synchronize()
        for i, (x, want) in enumerate(zip(outs, r)):
            got = host(x)
            assert np.all(np.isfinite(got) | ~np.isfinite(want)), f"{name} output {i}: NaN left by the fill"
            assert np.array_equal(got, want, equal_nan=True), f"{name} output {i} differs from the default stream's"


def test_concurrent_streams_share_no_state():
    """Two independent sets of calls (different inputs) interleaved on two
    side streams run concurrently and each gives bitwise the results of a
    run on its own: no entry point keeps device state between calls (the
    no-allocation backward, whose static scratch concurrent calls share by
    design, is left out)."""
    torch = need_gpu()
    sets = [[c for c in _calls(torch, seed) if c[0] != "fa_bwd_noalloc"] for seed in (0, 100)]
    refs = []
    for calls in sets:
        for _, outs, launch in calls:
            launch()
        torch.cuda.synchronize()
        refs.append([[host(x).copy() for x in outs] for _, outs, _ in calls])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    for calls, st in zip(sets, streams):
        with torch.cuda.stream(st):
            for _, outs, _ in calls:
                for x in outs:
                    x.fill_(float("nan"))
    for i in range(len(sets[0])):
        for calls, st in zip(sets, streams):
            with torch.cuda.stream(st):
                calls[i][2]()
    torch.cuda.synchronize()
    for k, (calls, ref) in enumerate(zip(sets, refs)):
        for (name, outs, _), r in zip(calls, ref):
            for j, (x, want) in enumerate(zip(outs, r)):
                assert np.array_equal(host(x), want, equal_nan=True), f"set {k} {name} output {j}"
        log(f"concurrent set {k} ok")
