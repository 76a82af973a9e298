#!/usr/bin/env python3
"""Benchmark of the tiled-attention hot path on one MI355X.

One step = fa_fwd + fa_bwd (a dQ launch that also forms Delta, then dK/dV) on the causal bf16
workload B=4, H=16, M=N=2048, D=128 with inputs already resident in HBM.
``value`` is that step's throughput in TFLOP/s under the Triton tutorial's
flop convention (forward 4*B*H*M*N*D, halved for causal; backward 2.5x the
forward).  The same JSON line carries:

* ``roofline`` for the dominant kernel of the step (its average launch time
  from HIP events recorded on the launch stream over a timed loop), against
  MI355X's dense bf16 MFMA peak of 2.5 PFLOP/s;
* ``components``: per-kernel times of the step and the other workloads of
  the hot path -- non-causal bf16 B1 H32 8192 D128, the fused JVP (fp16 B4 H16
  1024 D64, causal and not), piecewise attention (fp16 B2 H16 4096 D64, w =
  1024), the FP8 forward, head dims 16 and 256 (causal bf16 B1 H16 2048), the
  residual merge (bf16 32768 x 4096, in HBM GB/s against 8 TB/s) and the
  N-way merge;
* ``cpu_baseline``: the fp64 numpy oracle timed on the host on a bounded
  sample of the same workload (a few whole heads).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
HEADLINE = "causal_bf16_b4h16_s2048_d128"
METRIC = "attention fwd/bwd TFLOP/s + % bf16 MFMA peak; residual-merge HBM GB/s"


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """Average duration of repeated launches, from HIP events recorded on the
    stream the library launches on (torch's current stream).  Before timing,
    the launch is repeated for WARM_S seconds: after the host-side input
    set-up of a workload the GPU's clocks have dropped, and they take about
    0.2 s of work to ramp up again (a loop of a hundred 100 us launches timed
    right away reads 10-20% slow)."""

    WARM_S = 0.3

    def __init__(self, torch):
        self.torch = torch

    def avg_ms(self, fn, iters, warmup=2):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < self.WARM_S:
            for _ in range(10):
                fn()
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(iters):
            fn()
        end.record()
        end.synchronize()
        return start.elapsed_time(end) / iters


def attn_setup(torch, wl, names):
    from attention_fa2_tiles_amd.inputs import attn_inputs
    from attention_fa2_tiles_amd.devbuf import dev
    t = attn_inputs(wl, names)
    return t, {n: dev(t[n]) for n in names}


def attn_buffers(torch, wl, d, bwd=True):
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.devbuf import empty, empty_f32
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    buf = {"o": empty((B, H, M, D), wl.dtype), "lse": empty_f32((B, H, M)), "delta": empty_f32((B, H, M))}
    if bwd:
        for n in ("dq", "dk", "dv"):
            buf[n] = empty((B, H, M if n == "dq" else N, D), wl.dtype)
        nb = lib.fa_bwd_workspace_size(B, H, M, N, D, wl.dtype)
        buf["ws"] = torch.empty(nb, dtype=torch.uint8, device="cuda")
        buf["ws_bytes"] = nb
    return buf


def attn_calls(wl, d, b):
    from attention_fa2_tiles_amd import lib
    B, H, M, N, D, c, s = wl.B, wl.H, wl.M, wl.N, wl.D, wl.causal, wl.sm_scale
    q, k, v, do = d["q"], d["k"], d["v"], d["do"]
    return {
        "fwd": lambda: lib.fa_fwd(wl.dtype, q, k, v, b["o"], b["lse"], B, H, M, N, D, c, s),
        "bwd": lambda: lib.fa_bwd(wl.dtype, q, k, v, b["o"], do, b["lse"], b["dq"], b["dk"], b["dv"],
                                  b["ws"], b["ws_bytes"], B, H, M, N, D, c, s),
        "delta": lambda: lib.fa_bwd_delta(wl.dtype, b["o"], do, None, b["delta"], B, H, M, D),
        "dkdv": lambda: lib.fa_bwd_dkdv(wl.dtype, q, k, v, do, b["lse"], b["delta"], b["dk"], b["dv"],
                                        B, H, M, N, D, c, s),
        # the launch fa_bwd makes for 16-bit dtypes: the dQ pass forming Delta
        "dq": lambda: lib.fa_bwd_dq_delta(wl.dtype, q, k, v, b["o"], do, b["lse"], None, b["delta"], b["dq"],
                                          B, H, M, N, D, c, s),
    }


def kernel_work(wl):
    """Algorithmic work per launch of each kernel of one step.

    GEMM-equivalents of 2*M*N*D flops per head (halved when causal): the
    forward does two (S, PV); the backward's five (S recomputed, dP, dV, dK,
    dQ -- the 2.5x of the flop convention) are split as four for the dK/dV
    kernel and one (dQ) for the dQ kernel, which also recomputes S and dP
    and forms Delta (reading O).  The standalone Delta kernel (fp32 path) is
    bandwidth-bound: it reads O and dO and writes one fp32 per row."""
    g = 2.0 * wl.B * wl.H * wl.M * wl.N * wl.D * (0.5 if wl.causal else 1.0)
    es = 4 if wl.dtype == 0 else 2
    return {
        "fwd": ("mfma", 2 * g),
        "dkdv": ("mfma", 4 * g),
        "dq": ("mfma", 1 * g),
        "delta": ("hbm", 2.0 * wl.B * wl.H * wl.M * wl.D * es + 4.0 * wl.B * wl.H * wl.M),
    }


KERNEL_LABELS = {
    "fwd": "forward (fa_fwd)",
    "dkdv": "dK/dV pass of the backward (4 of its 5 counted GEMM-equivalents)",
    "dq": "dQ pass of the backward (forms Delta; 1 of its 5 counted GEMM-equivalents)",
}


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "fwd": ["attention_fa2_tiles_amd/csrc/attn_fwd.hip", "attention_fa2_tiles_amd/csrc/common.h"],
    "dkdv": ["attention_fa2_tiles_amd/csrc/attn_bwd.hip", "attention_fa2_tiles_amd/csrc/bwd_common.h",
             "attention_fa2_tiles_amd/csrc/common.h"],
    "dq": ["attention_fa2_tiles_amd/csrc/attn_bwd.hip", "attention_fa2_tiles_amd/csrc/bwd_common.h",
           "attention_fa2_tiles_amd/csrc/common.h"],
    "delta": ["attention_fa2_tiles_amd/csrc/attn_bwd.hip"],
    "merge_fwd": ["attention_fa2_tiles_amd/csrc/merge.hip", "attention_fa2_tiles_amd/csrc/common.h"],
    "merge_bwd": ["attention_fa2_tiles_amd/csrc/merge.hip", "attention_fa2_tiles_amd/csrc/common.h"],
    "lse_merge_fwd": ["attention_fa2_tiles_amd/csrc/lse_merge.hip", "attention_fa2_tiles_amd/csrc/common.h"],
    "lse_merge_bwd": ["attention_fa2_tiles_amd/csrc/lse_merge.hip", "attention_fa2_tiles_amd/csrc/common.h"],
}
MERGE_NAME = "merge_bf16_rows32768_d4096"


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_digest") != source_digest(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def bench_headline(torch, args, timer):
    from attention_fa2_tiles_amd.inputs import WORKLOADS
    wl = WORKLOADS[HEADLINE]
    progress(f"inputs for {wl.name}")
    _, d = attn_setup(torch, wl, ("q", "k", "v", "do"))
    b = attn_buffers(torch, wl, d)
    calls = attn_calls(wl, d, b)

    def step():
        calls["fwd"]()
        calls["bwd"]()

    progress(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # then the same clock ramp as every per-kernel loop (Timer.WARM_S): with a
    # handful of warm-up steps the clocks are still low when timing starts
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < Timer.WARM_S:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    progress(f"timing {args.steps} steps")
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    flops = wl.fwd_flops() + wl.bwd_flops()
    tflops = flops / (ms_step * 1e-3) / 1e12

    progress("per-kernel timing")
    iters = max(args.steps, 10)
    per = {k: timer.avg_ms(calls[k], iters) for k in ("fwd", "dq", "dkdv")}
    work = kernel_work(wl)
    kernels = {}
    for k, ms in per.items():
        bound, amount = work[k]
        if bound == "mfma":
            ach = amount / (ms * 1e-3) / 1e12
            kernels[k] = {"ms": round(ms, 5), "TFLOP/s": round(ach, 2),
                          "frac_bf16_peak": round(ach / PEAK_BF16_TFLOPS, 4)}
        else:
            ach = amount / (ms * 1e-3) / 1e9
            kernels[k] = {"ms": round(ms, 5), "GB/s": round(ach, 1), "frac_hbm_peak": round(ach / PEAK_HBM_GBPS, 4)}
    dominant = max(("fwd", "dkdv", "dq"), key=lambda k: per[k])
    bound, amount = work[dominant]
    achieved = amount / (per[dominant] * 1e-3) / 1e12
    roofline = {
        "kernel": dominant,
        "scope": f"one kernel: the {KERNEL_LABELS[dominant]}, the longest of the step; "
                 "the whole forward and backward are in step_fracs",
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": measured_traffic(HEADLINE, dominant),
        "avg_launch_ms": round(per[dominant], 5),
        "algorithmic_flops_per_launch": amount,
    }
    fwd_tf = wl.fwd_flops() / (per["fwd"] * 1e-3) / 1e12
    bwd_ms = timer.avg_ms(calls["bwd"], iters)
    bwd_tf = wl.bwd_flops() / (bwd_ms * 1e-3) / 1e12
    roofline["step_fracs"] = {"fwd": round(fwd_tf / PEAK_BF16_TFLOPS, 4), "bwd": round(bwd_tf / PEAK_BF16_TFLOPS, 4)}
    summary = {
        "fwd_TFLOP/s": round(fwd_tf, 2), "fwd_frac_peak": round(fwd_tf / PEAK_BF16_TFLOPS, 4),
        "bwd_TFLOP/s": round(bwd_tf, 2), "bwd_frac_peak": round(bwd_tf / PEAK_BF16_TFLOPS, 4),
        "bwd_ms": round(bwd_ms, 5), "kernels": kernels,
    }
    return wl, ms_step, tflops, wall, roofline, summary


def bench_attention_other(torch, timer, name, iters):
    from attention_fa2_tiles_amd.inputs import WORKLOADS
    wl = WORKLOADS[name]
    progress(f"component {name}")
    _, d = attn_setup(torch, wl, ("q", "k", "v", "do"))
    b = attn_buffers(torch, wl, d)
    calls = attn_calls(wl, d, b)
    calls["fwd"]()
    f_ms = timer.avg_ms(calls["fwd"], iters)
    b_ms = timer.avg_ms(calls["bwd"], iters)
    f_tf = wl.fwd_flops() / (f_ms * 1e-3) / 1e12
    b_tf = wl.bwd_flops() / (b_ms * 1e-3) / 1e12
    del d, b
    torch.cuda.empty_cache()
    return {"fwd_ms": round(f_ms, 4), "fwd_TFLOP/s": round(f_tf, 2), "fwd_frac_peak": round(f_tf / PEAK_BF16_TFLOPS, 4),
            "bwd_ms": round(b_ms, 4), "bwd_TFLOP/s": round(b_tf, 2), "bwd_frac_peak": round(b_tf / PEAK_BF16_TFLOPS, 4)}


def bench_tiny_f32(torch, timer, iters):
    """The tiny fp32 workload (B1 H2 128^2 D64, non-causal), reported without
    a target: fp32 runs the generic vector-ALU kernels in true fp32, and at
    8.4 MFLOP per forward the kernels are latency-bound (each of the 256
    query rows is walked key by key by one lane group).  Rates are against
    the fp32 vector peak."""
    from attention_fa2_tiles_amd.inputs import WORKLOADS
    wl = WORKLOADS["tiny_f32"]
    progress("component tiny_f32")
    _, d = attn_setup(torch, wl, ("q", "k", "v", "do"))
    b = attn_buffers(torch, wl, d)
    calls = attn_calls(wl, d, b)
    calls["fwd"]()
    f_ms = timer.avg_ms(calls["fwd"], iters)
    b_ms = timer.avg_ms(calls["bwd"], iters)
    f_tf = wl.fwd_flops() / (f_ms * 1e-3) / 1e12
    b_tf = wl.bwd_flops() / (b_ms * 1e-3) / 1e12
    del d, b
    return {"workload": "fp32 B1 H2 M=N=128 D64 non-causal", "fwd_us": round(f_ms * 1e3, 2),
            "fwd_TFLOP/s": round(f_tf, 4), "bwd_us": round(b_ms * 1e3, 2), "bwd_TFLOP/s": round(b_tf, 4),
            "frac_fp32_vector_peak": [round(f_tf / PEAK_FP32_TFLOPS, 5), round(b_tf / PEAK_FP32_TFLOPS, 5)],
            "kernels": "generic (vector ALU, fp32)"}


def bench_jvp(torch, timer, name, iters):
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import WORKLOADS
    from attention_fa2_tiles_amd.devbuf import empty, empty_f32
    wl = WORKLOADS[name]
    progress(f"component {name}")
    names = ("q", "k", "v", "tq", "tk", "tv")
    _, d = attn_setup(torch, wl, names)
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o, to, lse = empty((B, H, M, D), wl.dtype), empty((B, H, M, D), wl.dtype), empty_f32((B, H, M))
    ms = timer.avg_ms(lambda: lib.fa_fwd_jvp(wl.dtype, *[d[n] for n in names], o, lse, to,
                                             B, H, M, N, D, wl.causal, wl.sm_scale), iters)
    tf = 3 * wl.fwd_flops() / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "counted_flops": "3 x forward"}


def bench_fp8(torch, timer, iters):
    """fa_fwd_fp8 on the causal headline shape (B4 H16 2048 D128), e5m2
    q, k, v^t, bf16 output."""
    import numpy as np
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import BF16, F8E5M2, WORKLOADS, AttnWorkload, attn_inputs
    from attention_fa2_tiles_amd.devbuf import empty, empty_f32
    base = WORKLOADS[HEADLINE]
    wl = AttnWorkload("fp8_causal_b4h16_s2048_d128", F8E5M2, base.B, base.H, base.M, base.N, base.D, True,
                      base.seed)
    progress(f"component {wl.name}")
    t = attn_inputs(wl, ("q", "k", "v"))
    q = torch.from_numpy(t["q"].storage).cuda()
    k = torch.from_numpy(t["k"].storage).cuda()
    vt = torch.from_numpy(np.ascontiguousarray(np.swapaxes(t["v"].storage, 2, 3))).cuda()
    del t
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o, lse = empty((B, H, M, D), BF16), empty_f32((B, H, M))
    ms = timer.avg_ms(lambda: lib.fa_fwd_fp8(BF16, q, k, vt, o, lse, B, H, M, N, D, 1, 0.0), iters)
    tf = wl.fwd_flops() / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
            "inputs": "e5m2 q, k, v (v transposed)", "output": "bf16"}


def bench_pw(torch, timer, iters):
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import PIECEWISE_W, WORKLOADS
    from attention_fa2_tiles_amd.devbuf import empty, empty_f32
    wl = WORKLOADS["piecewise_f16_b2h16_s4096_d64_w1024"]
    progress(f"component {wl.name}")
    names = ("q1", "k1", "q2", "k2", "v", "do")
    _, d = attn_setup(torch, wl, names)
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o, lse = empty((B, H, M, D), wl.dtype), empty_f32((B, H, M))
    g = [empty((B, H, M, D), wl.dtype) for _ in range(5)]
    nb = lib.pw_bwd_workspace_size(B, H, M, N, D, wl.dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    args = (B, H, M, N, D, wl.causal, wl.sm_scale, PIECEWISE_W)
    fwd = lambda: lib.pw_fwd(wl.dtype, *[d[n] for n in names[:5]], o, lse, *args)
    bwd = lambda: lib.pw_bwd(wl.dtype, *[d[n] for n in names[:5]], o, d["do"], lse, *g, ws, nb, *args)
    fwd()
    f_ms = timer.avg_ms(fwd, iters)
    b_ms = timer.avg_ms(bwd, iters)
    f_tf = wl.fwd_flops() / (f_ms * 1e-3) / 1e12
    b_tf = wl.bwd_flops() / (b_ms * 1e-3) / 1e12
    return {"fwd_ms": round(f_ms, 4), "fwd_TFLOP/s": round(f_tf, 2), "bwd_ms": round(b_ms, 4),
            "bwd_TFLOP/s": round(b_tf, 2), "counted_flops": "one QK^T per score"}


def bench_head_dims(torch, timer, iters):
    """The head dims at the ends of the supported range, causal bf16 B1 H16
    M=N=2048: D = 256 (the backward passes and the fused JVP run one wave
    per SIMD) and D = 16 (the D = 32 kernels over zero-padded rows), every
    call on the matrix cores.  Same flop convention as the headline."""
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import BF16, AttnWorkload
    from attention_fa2_tiles_amd.devbuf import empty, empty_f32
    out = {}
    for D in (256, 16):
        wl = AttnWorkload(f"causal_bf16_b1h16_s2048_d{D}", BF16, 1, 16, 2048, 2048, D, True, seed=6)
        progress(f"component {wl.name}")
        names = ("q", "k", "v", "do")
        _, d = attn_setup(torch, wl, names)
        b = attn_buffers(torch, wl, d)
        calls = attn_calls(wl, d, b)
        B, H, M, N = wl.B, wl.H, wl.M, wl.N
        to = empty((B, H, M, D), wl.dtype)
        jvp = lambda: lib.fa_fwd_jvp(wl.dtype, d["q"], d["k"], d["v"], d["q"], d["k"], d["v"], b["o"], b["lse"], to,
                                     B, H, M, N, D, wl.causal, wl.sm_scale)
        calls["fwd"]()
        n = max(3, iters // 4)
        f_ms = timer.avg_ms(calls["fwd"], n)
        b_ms = timer.avg_ms(calls["bwd"], n)
        j_ms = timer.avg_ms(jvp, n)
        tf = lambda flops, ms: flops / (ms * 1e-3) / 1e12
        out[f"d{D}"] = {
            "workload": wl.name,
            "fwd_ms": round(f_ms, 4), "fwd_TFLOP/s": round(tf(wl.fwd_flops(), f_ms), 2),
            "bwd_ms": round(b_ms, 4), "bwd_TFLOP/s": round(tf(wl.bwd_flops(), b_ms), 2),
            "jvp_ms": round(j_ms, 4), "jvp_TFLOP/s": round(tf(3 * wl.fwd_flops(), j_ms), 2),
            "kernels": "MFMA" if D == 256 else "MFMA (D = 32 tiles over zero-padded rows)",
        }
        del d, b, calls, to
        torch.cuda.empty_cache()
    return out


def bench_merge(torch, timer, iters):
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import MERGE_WORKLOAD, merge_inputs
    from attention_fa2_tiles_amd.devbuf import dev, empty, empty_f32
    wl = MERGE_WORKLOAD
    progress(f"component {wl.name}")
    t = merge_inputs(wl)
    x, y0, q, l0, gy, gl = (dev(t[n]) for n in ("x", "y0", "q", "l0", "gy", "gl"))
    del t
    R, D = wl.rows, wl.D
    y, lse = empty((R, D), wl.dtype), empty_f32((R,))
    gx, gy0, gq, gl0 = empty((R, D), wl.dtype), empty((R, D), wl.dtype), empty_f32((D,)), empty_f32((R,))
    nb = lib.resmerge_bwd_workspace_size(R, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    fwd = lambda: lib.resmerge_fwd(wl.dtype, x, q, y0, l0, y, lse, R, D, wl.eps)
    bwd = lambda: lib.resmerge_bwd(wl.dtype, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, ws, nb, R, D, wl.eps)
    f_ms = timer.avg_ms(fwd, iters)
    b_ms = timer.avg_ms(bwd, iters)
    f_gb = wl.fwd_bytes() / (f_ms * 1e-3) / 1e9
    b_gb = wl.bwd_bytes() / (b_ms * 1e-3) / 1e9
    return {"fwd_ms": round(f_ms, 4), "fwd_GB/s": round(f_gb, 1), "fwd_frac_hbm": round(f_gb / PEAK_HBM_GBPS, 4),
            "bwd_ms": round(b_ms, 4), "bwd_GB/s": round(b_gb, 1), "bwd_frac_hbm": round(b_gb / PEAK_HBM_GBPS, 4),
            "fwd_bytes": wl.fwd_bytes(), "bwd_bytes": wl.bwd_bytes(),
            "fwd_traffic": measured_traffic(MERGE_NAME, "merge_fwd"),
            "bwd_traffic": measured_traffic(MERGE_NAME, "merge_bwd")}


def bench_lse_merge(torch, timer, iters):
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import LSE_MERGE_WORKLOAD, lse_merge_inputs
    from attention_fa2_tiles_amd.devbuf import dev, empty, empty_f32
    wl = LSE_MERGE_WORKLOAD
    progress(f"component {wl.name}")
    t = lse_merge_inputs(wl)
    ys, lses, gy, gl = (dev(t[n]) for n in ("ys", "lses", "gy", "gl"))
    del t
    S, R, D = wl.S, wl.rows, wl.D
    y, lse = empty((R, D), wl.dtype), empty_f32((R,))
    gys, glses = empty((S, R, D), wl.dtype), empty_f32((S, R))
    fwd = lambda: lib.lse_merge_fwd(wl.dtype, ys, lses, y, lse, S, R, D)
    bwd = lambda: lib.lse_merge_bwd(wl.dtype, ys, lses, gy, gl, gys, glses, S, R, D)
    f_ms = timer.avg_ms(fwd, iters)
    b_ms = timer.avg_ms(bwd, iters)
    f_gb = wl.fwd_bytes() / (f_ms * 1e-3) / 1e9
    b_gb = wl.bwd_bytes() / (b_ms * 1e-3) / 1e9
    return {"fwd_ms": round(f_ms, 4), "fwd_GB/s": round(f_gb, 1), "fwd_frac_hbm": round(f_gb / PEAK_HBM_GBPS, 4),
            "bwd_ms": round(b_ms, 4), "bwd_GB/s": round(b_gb, 1), "bwd_frac_hbm": round(b_gb / PEAK_HBM_GBPS, 4),
            "fwd_bytes": wl.fwd_bytes(), "bwd_bytes": wl.bwd_bytes(),
            "fwd_traffic": measured_traffic(wl.name, "lse_merge_fwd"),
            "bwd_traffic": measured_traffic(wl.name, "lse_merge_bwd")}


def cpu_baseline(target_s):
    """The fp64 oracle, as it stands, on whole heads of the headline workload."""
    import numpy as np
    import oracle
    from attention_fa2_tiles_amd.inputs import WORKLOADS, AttnWorkload, attn_inputs
    wl = WORKLOADS[HEADLINE]
    progress("cpu baseline (fp64 oracle)")
    one = AttnWorkload("sample", wl.dtype, 1, 1, wl.M, wl.N, wl.D, wl.causal, wl.seed)
    per_head = one.fwd_flops() + one.bwd_flops()

    def run(nheads):
        w = AttnWorkload("sample", wl.dtype, 1, nheads, wl.M, wl.N, wl.D, wl.causal, wl.seed)
        t = attn_inputs(w)
        f = {n: t[n].f64 for n in ("q", "k", "v", "do")}
        t0 = time.perf_counter()
        oracle.attn_fwd(f["q"], f["k"], f["v"], wl.causal, wl.scale())
        oracle.attn_bwd(f["q"], f["k"], f["v"], f["do"], wl.causal, wl.scale())
        return time.perf_counter() - t0

    t1 = run(1)
    n = int(max(1, min(wl.B * wl.H, round(target_s / max(t1, 1e-3)))))
    tn = run(n) if n > 1 else t1
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            threads = max(p.get("num_threads", 1) for p in info)
    except Exception:
        pass
    del np
    return {"value": round(n * per_head / tn / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fa_fwd + fa_bwd fp64 numpy oracle on {n} of {wl.B * wl.H} heads of {wl.name} "
                      f"(B=1, H={n}); {tn:.1f} s wall",
            "seconds": round(tn, 2)}


def profile_mode(torch):
    """Launch each kernel of the headline step, the residual merge, the N-way
    merge and the other attention workloads a few times, then copy 256 MiB
    device-to-device; rocprofv3 --pmc runs wrap this to count HBM bytes and
    other counters per dispatch, and the copy's counter value per byte is
    the calibration."""
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import (LSE_MERGE_WORKLOAD, MERGE_WORKLOAD, WORKLOADS, lse_merge_inputs,
                                                merge_inputs)
    from attention_fa2_tiles_amd.devbuf import dev, empty, empty_f32
    wl = WORKLOADS[HEADLINE]
    _, d = attn_setup(torch, wl, ("q", "k", "v", "do"))
    b = attn_buffers(torch, wl, d)
    calls = attn_calls(wl, d, b)
    calls["fwd"]()
    for k in ("fwd", "dq", "dkdv"):
        for _ in range(3):
            calls[k]()
        torch.cuda.synchronize()
        progress(f"profiled {k}")
    del d, b, calls
    mw = MERGE_WORKLOAD
    t = merge_inputs(mw)
    x, y0, q, l0, gy, gl = (dev(t[n]) for n in ("x", "y0", "q", "l0", "gy", "gl"))
    del t
    R, D = mw.rows, mw.D
    y, lse = empty((R, D), mw.dtype), empty_f32((R,))
    gx, gy0, gq, gl0 = empty((R, D), mw.dtype), empty((R, D), mw.dtype), empty_f32((D,)), empty_f32((R,))
    nb = lib.resmerge_bwd_workspace_size(R, D)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        lib.resmerge_fwd(mw.dtype, x, q, y0, l0, y, lse, R, D, mw.eps)
    torch.cuda.synchronize()
    progress("profiled merge fwd")
    for _ in range(3):
        lib.resmerge_bwd(mw.dtype, x, q, y0, l0, gy, gl, gx, gq, gy0, gl0, ws, nb, R, D, mw.eps)
    torch.cuda.synchronize()
    progress("profiled merge bwd")
    del x, y0, q, l0, gy, gl, y, lse, gx, gy0, gq, gl0, ws
    lw = LSE_MERGE_WORKLOAD
    t = lse_merge_inputs(lw)
    ys, lses, gy, gl = (dev(t[n]) for n in ("ys", "lses", "gy", "gl"))
    del t
    y, lse = empty((lw.rows, lw.D), lw.dtype), empty_f32((lw.rows,))
    gys, glses = empty((lw.S, lw.rows, lw.D), lw.dtype), empty_f32((lw.S, lw.rows))
    for _ in range(3):
        lib.lse_merge_fwd(lw.dtype, ys, lses, y, lse, lw.S, lw.rows, lw.D)
    torch.cuda.synchronize()
    progress("profiled lse_merge fwd")
    for _ in range(3):
        lib.lse_merge_bwd(lw.dtype, ys, lses, gy, gl, gys, glses, lw.S, lw.rows, lw.D)
    torch.cuda.synchronize()
    progress("profiled lse_merge bwd")
    del ys, lses, gy, gl, y, lse, gys, glses
    profile_other_attention(torch)
    torch.cuda.empty_cache()
    # calibration: an elementwise copy (dst = -src) of COPY_BYTES, launched
    # over the whole device like the kernels above
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    progress("profiled copy")


COPY_BYTES = 256 << 20


def profile_other_attention(torch):
    """profile_mode's launches of the other attention workloads, for their
    counters: the fused JVP (fp16 B4 H16 1024^2 D64, causal and not),
    piecewise attention forward and backward (fp16 B2 H16 4096^2 D64,
    w = 1024, causal) and the FP8 forward (causal B4 H16 2048^2 D128)."""
    import numpy as np
    from attention_fa2_tiles_amd import lib
    from attention_fa2_tiles_amd.inputs import BF16, F8E5M2, PIECEWISE_W, WORKLOADS, AttnWorkload, attn_inputs
    from attention_fa2_tiles_amd.devbuf import empty, empty_f32
    names = ("q", "k", "v", "tq", "tk", "tv")
    for name in ("jvp_f16_b4h16_s1024_d64_causal", "jvp_f16_b4h16_s1024_d64"):
        wl = WORKLOADS[name]
        _, d = attn_setup(torch, wl, names)
        B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
        o, to, lse = empty((B, H, M, D), wl.dtype), empty((B, H, M, D), wl.dtype), empty_f32((B, H, M))
        for _ in range(3):
            lib.fa_fwd_jvp(wl.dtype, *[d[n] for n in names], o, lse, to, B, H, M, N, D, wl.causal, wl.sm_scale)
        torch.cuda.synchronize()
        progress(f"profiled {name}")
        del d, o, to, lse
    wl = WORKLOADS["piecewise_f16_b2h16_s4096_d64_w1024"]
    names = ("q1", "k1", "q2", "k2", "v", "do")
    _, d = attn_setup(torch, wl, names)
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o, lse = empty((B, H, M, D), wl.dtype), empty_f32((B, H, M))
    g = [empty((B, H, M, D), wl.dtype) for _ in range(5)]
    nb = lib.pw_bwd_workspace_size(B, H, M, N, D, wl.dtype)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    args = (B, H, M, N, D, wl.causal, wl.sm_scale, PIECEWISE_W)
    for _ in range(3):
        lib.pw_fwd(wl.dtype, *[d[n] for n in names[:5]], o, lse, *args)
    for _ in range(3):
        lib.pw_bwd(wl.dtype, *[d[n] for n in names[:5]], o, d["do"], lse, *g, ws, nb, *args)
    torch.cuda.synchronize()
    progress(f"profiled {wl.name}")
    del d, o, lse, g, ws
    base = WORKLOADS[HEADLINE]
    wl = AttnWorkload("fp8_causal_b4h16_s2048_d128", F8E5M2, base.B, base.H, base.M, base.N, base.D, True, base.seed)
    t = attn_inputs(wl, ("q", "k", "v"))
    q = torch.from_numpy(t["q"].storage).cuda()
    k = torch.from_numpy(t["k"].storage).cuda()
    vt = torch.from_numpy(np.ascontiguousarray(np.swapaxes(t["v"].storage, 2, 3))).cuda()
    del t
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    o, lse = empty((B, H, M, D), BF16), empty_f32((B, H, M))
    for _ in range(3):
        lib.fa_fwd_fp8(BF16, q, k, vt, o, lse, B, H, M, N, D, 1, 0.0)
    torch.cuda.synchronize()
    progress(f"profiled {wl.name}")
    del q, k, vt, o, lse

# kernel-name fragments (mangled) of the launches profile_mode makes
PROFILED = {
    "fwd": ("causal_bf16_b4h16_s2048_d128", "attn_fwd_pipe_kernelIDF16bLi128ELi0ELb1ELb0"),
    "dq": ("causal_bf16_b4h16_s2048_d128", "attn_dq_kernelIDF16bLi128ELi0ELb1ELb0"),
    "dkdv": ("causal_bf16_b4h16_s2048_d128", "attn_dkdv_kernelIDF16bLi128ELi0ELb1ELb0"),
    "merge_fwd": ("merge_bf16_rows32768_d4096", "N_116merge_fwd_kernelIDF16b"),
    "merge_bwd": ("merge_bf16_rows32768_d4096", "N_116merge_bwd_kernelIDF16b"),
    "lse_merge_fwd": ("lse_merge_bf16_s4_rows131072_d128", "lse_merge_fwd_small_kernelIDF16b"),
    "lse_merge_bwd": ("lse_merge_bf16_s4_rows131072_d128", "lse_merge_bwd_small_kernelIDF16b"),
    # counters only (no traffic record)
    "jvp_causal": (None, "attn_fwd_kernelIDF16_Li64ELi1ELb1ELb0"),
    "jvp": (None, "attn_fwd_kernelIDF16_Li64ELi1ELb0ELb0"),
    "pw_fwd": (None, "attn_fwd_pipe_kernelIDF16_Li64ELi2ELb1ELb0"),
    "pw_dq": (None, "attn_dq_kernelIDF16_Li64ELi2ELb1ELb0"),
    "pw_dkdv": (None, "attn_dkdv_kernelIDF16_Li64ELi2ELb1ELb0"),
    "fp8_fwd": (None, "attn_fwd_fp8_kernelIDF16bLi128ELb1ELb0"),
    "copy": (None, "neg"),
}
XCDS, SIMDS = 8, 1024   # MI355X: GRBM_GUI_ACTIVE sums its 8 XCDs; 256 CUs x 4 SIMDs


def read_counters(dirs):
    """{key: {counter: [value per dispatch, in dispatch order]}} from the
    counter_collection csv files of rocprofv3 --pmc runs of profile_mode."""
    import csv
    import glob
    out = {}
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            per = {}
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    key = next((k for k, (_, pat) in PROFILED.items() if pat in row["Kernel_Name"]), None)
                    if key is None:
                        continue
                    i = int(row["Dispatch_Id"])
                    disp = per.setdefault((key, row["Counter_Name"]), {})
                    disp[i] = disp.get(i, 0.0) + float(row["Counter_Value"])
                    per.setdefault((key, "duration_ns"), {})[i] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
            for (key, name), disp in per.items():
                out.setdefault(key, {})[name] = [disp[i] for i in sorted(disp)]
    return out


def steady(vals):
    """Mean over dispatches, leaving out the first (cold clocks and caches)
    when there are several."""
    v = vals[1:] if len(vals) > 1 else vals
    return sum(v) / len(v)


def summarize_traffic(fetch_dir, write_dir):
    """Scale FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what they read
    for the COPY_BYTES copy, and record HBM bytes per launch, with the digest
    of each kernel's sources, in profiles/traffic.json."""
    fetch = {k: steady(c["FETCH_SIZE"]) for k, c in read_counters([fetch_dir]).items() if "FETCH_SIZE" in c}
    write = {k: steady(c["WRITE_SIZE"]) for k, c in read_counters([write_dir]).items() if "WRITE_SIZE" in c}
    fs, ws = COPY_BYTES / (fetch["copy"] * 1024), COPY_BYTES / (write["copy"] * 1024)
    print(f"calibration copy of {COPY_BYTES >> 20} MiB: FETCH_SIZE {fetch['copy']:.0f} KiB, "
          f"WRITE_SIZE {write['copy']:.0f} KiB -> scale {fs:.4f} (fetch), {ws:.4f} (write)\n")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    print("| kernel | workload | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled HBM MiB / launch |")
    print("|---|---|---|---|---|")
    for key, (wl, _) in PROFILED.items():
        if wl is None or key not in fetch or key not in write:
            continue
        b = fetch[key] * 1024 * fs + write[key] * 1024 * ws
        data.setdefault(wl, {})[key] = {
            "bytes_per_launch": int(round(b)), "fetch_kib": fetch[key], "write_kib": write[key],
            "fetch_scale": fs, "write_scale": ws, "source_digest": source_digest(KERNEL_SOURCES[key])}
        print(f"| {key} | {wl} | {fetch[key]:.0f} | {write[key]:.0f} | {b / 2**20:.1f} |")
    with open(path, "w") as f:
        json.dump(data, f, indent=1)


def summarize_counters(dirs):
    """Per kernel, the steady mean of every counter collected, and where the
    counters are there: GPU cycles (GRBM_GUI_ACTIVE / 8 XCDs) and the clock
    they imply over the dispatch's duration (duration_ns), the fraction
    of SIMD-cycles the MFMA pipes were busy, and LDS instructions' share of
    the waves' active cycles."""
    data = read_counters(dirs)
    for key, ctr in data.items():
        if key == "copy":
            continue
        print(f"### {key}\n\n| counter | mean per dispatch |\n|---|---|")
        for name in sorted(ctr):
            print(f"| {name} | {steady(ctr[name]):.6g} |")
        m = {n: steady(v) for n, v in ctr.items()}
        if "GRBM_GUI_ACTIVE" in m:
            cyc = m["GRBM_GUI_ACTIVE"] / XCDS
            print(f"| (derived) GPU cycles per dispatch | {cyc:.6g} |")
            print(f"| (derived) shader clock, GHz (cycles / dispatch duration) | {cyc / m['duration_ns']:.3f} |")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                print(f"| (derived) MFMA busy, share of SIMD-cycles | {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * SIMDS):.4f} |")
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_LDS_IDX_ACTIVE" in m and m["SQ_LDS_IDX_ACTIVE"]:
            print(f"| (derived) LDS bank-conflict cycles / LDS active cycles | "
                  f"{m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.4f} |")
        print()


def summarize_trace(trace_dir):
    """Markdown table of a rocprofv3 --kernel-trace --stats run's per-kernel
    durations."""
    import csv
    import glob
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)[0]
    print("| kernel | calls | avg us | min us | max us |\n|---|---|---|---|---|")
    with open(f) as fh:
        for row in csv.DictReader(fh):
            print(f"| `{row['Name'][:100]}` | {row['Calls']} | {float(row['AverageNs']) / 1e3:.1f} | "
                  f"{float(row['MinNs']) / 1e3:.1f} | {float(row['MaxNs']) / 1e3:.1f} |")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # a few hundred warm-up steps (~0.2 s): the GPU's clocks need that long to
    # ramp up, and timings taken earlier read up to ~20% slow
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-components", action="store_true", help="time only the headline step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--profile", action="store_true",
                    help="counter-collection mode: a few launches of each kernel of the step and of the merge, "
                         "then an elementwise copy of 256 MiB (the byte-count calibration), no timing output")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="host only: turn the FETCH_SIZE and WRITE_SIZE --pmc runs of --profile into "
                         "profiles/traffic.json and print the table")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="host only: per-kernel table of the --pmc runs of --profile in DIR...")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="host only: per-kernel table of a rocprofv3 --kernel-trace --stats run")
    args = ap.parse_args()
    if args.summarize_traffic or args.summarize_counters or args.summarize_trace:
        if args.summarize_traffic:
            summarize_traffic(*args.summarize_traffic)
        if args.summarize_counters:
            summarize_counters(args.summarize_counters)
        if args.summarize_trace:
            summarize_trace(args.summarize_trace)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(attention heads and merge rows would shard across GPUs with no exchange; "
              "see the design notes).", file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: WORLD_SIZE > 1 is not supported (single-GPU build)", file=sys.stderr)
        sys.exit(2)

    import torch
    from attention_fa2_tiles_amd import lib
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    lib.load()
    torch.cuda.set_device(0)
    timer = Timer(torch)

    if args.profile:
        profile_mode(torch)
        return

    wl, ms_step, tflops, wall, roofline, summary = bench_headline(torch, args, timer)
    components = {HEADLINE: summary}
    if not args.no_components:
        iters = max(5, min(args.steps, 20))
        components["noncausal_bf16_b1h32_s8192_d128"] = bench_attention_other(
            torch, timer, "noncausal_bf16_b1h32_s8192_d128", max(3, iters // 2))
        components["jvp_f16_b4h16_s1024_d64_causal"] = bench_jvp(torch, timer, "jvp_f16_b4h16_s1024_d64_causal", iters)
        components["jvp_f16_b4h16_s1024_d64"] = bench_jvp(torch, timer, "jvp_f16_b4h16_s1024_d64", iters)
        components["piecewise_f16_b2h16_s4096_d64_w1024"] = bench_pw(torch, timer, iters)
        components["fp8_causal_b4h16_s2048_d128"] = bench_fp8(torch, timer, iters)
        components["head_dims_causal_bf16_b1h16_s2048"] = bench_head_dims(torch, timer, iters)
        components["tiny_f32_b1h2_s128_d64"] = bench_tiny_f32(torch, timer, iters)
        components["merge_bf16_rows32768_d4096"] = bench_merge(torch, timer, iters)
        components["lse_merge_bf16_s4_rows131072_d128"] = bench_lse_merge(torch, timer, iters)
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "clock_warm_s": Timer.WARM_S,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "M": wl.M, "N": wl.N, "D": wl.D,
                   "causal": wl.causal, "sm_scale": float(wl.scale()), "step": "fa_fwd + fa_bwd",
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "components": components,
        "timed_wall_s": round(wall, 4),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
