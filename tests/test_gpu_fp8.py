"""GPU parity: fa_fwd_fp8 (float8 e5m2 q, k, v) against the fp64 oracle.

The oracle computes exact attention on the decoded e5m2 inputs.  The kernel
rounds P to float8 e4m3 for the P V product and normalises by the sum of the
unrounded P, so O is compared against the first-order bound of that
rounding: with w_j = P_ij / sum_j P_ij and each weight off by a relative
delta_j, |delta_j| <= 2^-4 (round to nearest with 3 mantissa bits), the
output moves by sum_j w_j delta_j v_j, at most 2^-4 sum_j w_j |v_jd|; the
output's own rounding (2^-8 relative for bf16, 2^-11 for fp16) and fp32
accumulation (1e-3) are added.
The LSE comes from the unrounded P and meets the 16-bit 1e-2 bar.
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


def check_fp8_output(tag, got, q, k, v, causal, c, out_dtype):
    ro, rl = oracle.attn_fwd(q, k, v, causal, c)
    P, _ = oracle.attn_probs(q, k, causal, c)
    # first-order bound of the e4m3 rounding of the weights, per element
    bound = 2.0 ** -4 * np.einsum("bhmn,bhnd->bhmd", P, np.abs(v))
    out_rel = 2.0 ** -8 if out_dtype == BF16 else 2.0 ** -11
    tol = bound + out_rel * np.abs(ro) + 1e-3
    err = np.abs(got - ro)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), (f"{tag}: |o - ref| exceeds the P-rounding bound at {worst}: "
                                f"err {err[worst]:.3e} > tol {tol[worst]:.3e} (max err {err.max():.3e})")
    log(f"{tag}: max |o - ref| {err.max():.3e}, max bound {tol.max():.3e}")
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
