"""GPU parity: fa_fwd_fp8 (float8 e5m2 q, k, v) against the fp64 oracle.

The oracle computes exact attention on the decoded e5m2 inputs.  The kernel
rounds its unnormalised weights p_j = exp2(s_j - m) (m: its running row
maximum, never above the true one) to float8 e4m3 for the P V product and
normalises by the sum of the unrounded p.  The error bound follows from
e4m3's rounding (3 mantissa bits, smallest normal 2^-6, subnormal spacing
2^-9, round to nearest):
  * p >= 2^-6 (normal): |round(p) - p| <= 2^-4 p;
  * p <  2^-6 (subnormal, or flushed to 0 below 2^-10): |round(p) - p| <=
    2^-10, an absolute error.
Dividing by the row sum l >= Z = sum_j exp(S_j - max S) (the running maximum
is never above the row's true maximum, so l is at least the sum taken
against that maximum) turns these into, per output element d,
    sum_j (2^-4 P_j + 2^-10 [r_j < 2^-6] / Z) |v_jd|,
where P_j is the exact weight and r_j = exp(S_j - max S) = P_j / max_j P_j
(a key with r_j >= 2^-6 has p >= 2^-6 whatever the running maximum was, so
only keys with r_j < 2^-6 can take the absolute term).  Added: fp32
arithmetic (2^-16 sum_j P_j |v_jd|, far above the fp32 roundings of the
scores, exponentials and sums) and the output's own rounding to the stored
dtype (half an ulp: 2^-8 relative for bf16, 2^-11 for fp16).  The LSE comes
from the unrounded p and meets the 16-bit 1e-2 bar.
"""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.inputs import BF16, F16, F8E5M2, AttnWorkload, attn_inputs
from gpu_util import check_guards, dev, guarded, guarded_f32, host, log, need_gpu
from tolerance import check_lse

pytestmark = pytest.mark.gpu


def run_fp8(out_dtype, wl, t):
    torch = need_gpu()
    B, H, M, N, D = wl.B, wl.H, wl.M, wl.N, wl.D
    q, k = dev(t["q"]), dev(t["k"])
    vt = torch.from_numpy(np.ascontiguousarray(np.swapaxes(t["v"].storage, 2, 3))).cuda()
    o = guarded((B, H, M, D), out_dtype)
    lse = guarded_f32((B, H, M))
    lib.fa_fwd_fp8(out_dtype, q, k, vt, o, lse, B, H, M, N, D, wl.causal, wl.sm_scale)
    torch.cuda.synchronize()
    res = {"o": host(o), "lse": host(lse)}
    check_guards()
    return res


def fp8_output_bound(P, v, out_dtype, ref):
    """Per-element bound of |o - ref| for the e4m3 rounding of the weights
    (see the module docstring); P [B,H,M,N] exact weights, v [B,H,N,D]."""
    av = np.abs(v)
    pmax = P.max(axis=-1, keepdims=True)
    Z = np.where(pmax > 0, 1.0 / np.where(pmax > 0, pmax, 1.0), 1.0)   # sum_j exp(S_j - max S)
    r = np.where(pmax > 0, P / np.where(pmax > 0, pmax, 1.0), 1.0)     # exp(S_j - max S)
    sub = (r < 2.0 ** -6) & (P > 0)
    rel = np.einsum("bhmn,bhnd->bhmd", P, av)
    absolute = np.einsum("bhmn,bhnd->bhmd", sub / Z, av)
    bound = (2.0 ** -4 + 2.0 ** -16) * rel + 2.0 ** -10 * absolute
    out_rel = 2.0 ** -8 if out_dtype == BF16 else 2.0 ** -11
    return bound + out_rel * (np.abs(ref) + bound)


def check_fp8_output(tag, got, q, k, v, causal, c, out_dtype):
    ro, rl = oracle.attn_fwd(q, k, v, causal, c)
    P, _ = oracle.attn_probs(q, k, causal, c)
    tol = fp8_output_bound(P, v, out_dtype, ro)
    err = np.abs(got - ro)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"{tag}: |o - ref| exceeds the P-rounding bound at {worst}: "
                                f"err {err[worst]:.3e} > tol {tol[worst]:.3e} (max err {err.max():.3e})")
    ratio = np.max(err[tol > 0] / tol[tol > 0]) if np.any(tol > 0) else 0.0
    log(f"{tag}: max |o - ref| {err.max():.3e}, max bound {tol.max():.3e}, max err/bound {ratio:.3f}")
    return rl


CASES = [
    # out dtype, B, H, M, N, D, causal
    (BF16, 1, 2, 256, 256, 128, True),
    (BF16, 1, 2, 256, 256, 128, False),
    (F16, 2, 2, 192, 192, 64, True),
    (F16, 1, 2, 200, 144, 64, True),      # ragged M, N a multiple of 16
    (BF16, 1, 2, 130, 208, 128, False),   # partial last key block visited first
    (BF16, 1, 2, 320, 128, 64, True),     # M > N: rows that see no key
    (F16, 1, 1, 1, 16, 128, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_fp8_forward_parity(case):
    out_dtype, B, H, M, N, D, causal = case
    wl = AttnWorkload("fp8", F8E5M2, B, H, M, N, D, causal, seed=101 + M + N)
    log(f"fp8 forward parity {case}")
    t = attn_inputs(wl, ("q", "k", "v"))
    got = run_fp8(out_dtype, wl, t)
    q, k, v = (t[n].f64 for n in ("q", "k", "v"))
    rl = check_fp8_output(f"fp8{case}", got["o"], q, k, v, causal, wl.scale(), out_dtype)
    check_lse(f"fp8{case}.lse", got["lse"], rl, out_dtype)


def test_fp8_forward_benchmark_shape():
    """The shape the benchmark times (causal B4 H16 2048 D128, bf16 output):
    the whole output is finite and three heads (first, middle, last) meet
    the bound."""
    wl = AttnWorkload("fp8_causal_b4h16_s2048_d128", F8E5M2, 4, 16, 2048, 2048, 128, True, seed=2)
    log("fp8 forward parity at the benchmark shape")
    t = attn_inputs(wl, ("q", "k", "v"))
    got = run_fp8(BF16, wl, t)
    assert np.all(np.isfinite(got["o"])) and np.all(np.isfinite(got["lse"]))
    for b, h in ((0, 0), (1, 9), (3, 15)):
        f = {n: t[n].f64[b:b + 1, h:h + 1] for n in ("q", "k", "v")}
        rl = check_fp8_output(f"fp8 bench[b={b},h={h}]", got["o"][b:b + 1, h:h + 1], f["q"], f["k"], f["v"],
                              True, wl.scale(), BF16)
        check_lse(f"fp8 bench[b={b},h={h}].lse", got["lse"][b:b + 1, h:h + 1], rl, BF16)
