"""GPU parity on one very long head pair: attention (bf16 D128), the fused
JVP and piecewise attention (fp16 D64) with 32768 keys (causal) or 16384
(non-causal).

The forward walks up to 512 key blocks per query block (the running maximum
raised lazily many times over), the dK/dV pass up to 1024 query blocks per
key block, and a head spans 128 (64) query blocks.  The oracle checks exactly
what it can compute in seconds at this length:

* O, LSE and dQ (the JVP: tO and tLSE) on windows of 8 query rows at the
  start, the middle and the end of each head: a window of rows needs all
  keys (non-causal) or only the keys up to its last row (causal: the
  oracle's bottom-right alignment of 8 rows against those keys is the
  global diagonal, and keeps the piecewise rule's distances);
* causal: dK and dV (piecewise: dK1, dK2, dV) of the last 64 keys, which
  only the last 64 query rows reach (the oracle's backward over those rows
  and all keys is exact there);
* every output finite.
"""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd.inputs import BF16, F16, AttnWorkload, attn_inputs
from gpu_util import log
from test_gpu_attention import run_fwd_bwd
from tolerance import check_grad, check_lse, check_output

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_long_head_windows(causal):
    S = 32768 if causal else 16384
    wl = AttnWorkload("long", BF16, 1, 2, S, S, 128, causal, seed=91 + int(causal))
    log(f"long head {S}x{S}, causal={causal}: drawing inputs")
    t = attn_inputs(wl)
    got = run_fwd_bwd(wl, t)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values"
    c = wl.scale()
    r = 8
    for h in range(wl.H):
        f = {n: t[n].f64[:, h:h + 1] for n in ("q", "k", "v", "do")}
        for i0 in (0, S // 2 - r // 2, S - r):
            kend = i0 + r if causal else S
            qs, dos = f["q"][:, :, i0:i0 + r], f["do"][:, :, i0:i0 + r]
            ks, vs = f["k"][:, :, :kend], f["v"][:, :, :kend]
            ro, rl = oracle.attn_fwd(qs, ks, vs, causal, c)
            rdq, _, _ = oracle.attn_bwd(qs, ks, vs, dos, causal, c)
            tag = f"long[h={h}, rows {i0}..{i0 + r - 1}]"
            check_output(tag + ".o", got["o"][0, h, i0:i0 + r], ro[0, 0], BF16)
            check_lse(tag + ".lse", got["lse"][0, h, i0:i0 + r], rl[0, 0], BF16)
            check_grad(tag + ".dq", got["dq"][0, h, i0:i0 + r], rdq[0, 0], BF16)
        if causal:
            tail = 64
            _, rdk, rdv = oracle.attn_bwd(f["q"][:, :, S - tail:], f["k"], f["v"], f["do"][:, :, S - tail:], True, c)
            tag = f"long[h={h}, keys {S - tail}..{S - 1}]"
            check_grad(tag + ".dk", got["dk"][0, h, S - tail:], rdk[0, 0, S - tail:], BF16)
            check_grad(tag + ".dv", got["dv"][0, h, S - tail:], rdv[0, 0, S - tail:], BF16)
        log(f"long head {h} ok")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_long_head_jvp_windows(causal):
    """Fused JVP, fp16 B1 H2 D64 with 32768 (causal) or 16384 keys: O, LSE,
    tO and tLSE on row windows."""
    from test_gpu_jvp_piecewise import JVP_NAMES, run_jvp
    S = 32768 if causal else 16384
    wl = AttnWorkload("long_jvp", F16, 1, 2, S, S, 64, causal, seed=93 + int(causal))
    log(f"long head JVP {S}x{S}, causal={causal}")
    t = attn_inputs(wl, JVP_NAMES)
    got = run_jvp(wl, t)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values"
    c = wl.scale()
    r = 8
    for h in range(wl.H):
        f = {n: t[n].f64[:, h:h + 1] for n in JVP_NAMES}
        for i0 in (0, S // 2 - r // 2, S - r):
            kend = i0 + r if causal else S
            win = [f[n][:, :, i0:i0 + r] if n in ("q", "tq") else f[n][:, :, :kend] for n in JVP_NAMES]
            o, lse, to, tlse = oracle.attn_fwd_jvp(*win, causal, c)
            tag = f"long_jvp[h={h}, rows {i0}..{i0 + r - 1}]"
            check_output(tag + ".o", got["o"][0, h, i0:i0 + r], o[0, 0], F16)
            check_lse(tag + ".lse", got["lse"][0, h, i0:i0 + r], lse[0, 0], F16)
            check_grad(tag + ".to", got["to"][0, h, i0:i0 + r], to[0, 0], F16)
            check_grad(tag + ".tlse", got["tlse"][0, h, i0:i0 + r], tlse[0, 0], F16)


def test_long_head_piecewise_windows():
    """Piecewise attention, fp16 B1 H2 D64, 32768 keys, causal, w = 1024:
    O, LSE, dQ1 and dQ2 on row windows (the distance rule sees global
    indices: the window's alignment against keys up to its last row keeps
    them), dK1, dK2 and dV of the last 64 keys."""
    from test_gpu_jvp_piecewise import PW_NAMES, run_pw
    S, w = 32768, 1024
    wl = AttnWorkload("long_pw", F16, 1, 2, S, S, 64, True, seed=95)
    log(f"long head piecewise {S}x{S}, w={w}")
    t = attn_inputs(wl, PW_NAMES)
    got = run_pw(wl, t, w)
    for n, x in got.items():
        assert np.all(np.isfinite(x)), f"{n}: non-finite values"
    c = wl.scale()
    r = 8
    for h in range(wl.H):
        f = {n: t[n].f64[:, h:h + 1] for n in PW_NAMES}
        for i0 in (0, S // 2 - r // 2, S - r):
            kend = i0 + r
            win = [f[n][:, :, i0:i0 + r] if n in ("q1", "q2", "do") else f[n][:, :, :kend] for n in PW_NAMES]
            o, lse = oracle.pw_fwd(*win[:5], True, c, w)
            dq1, _, dq2, _, _ = oracle.pw_bwd(*win, True, c, w)
            tag = f"long_pw[h={h}, rows {i0}..{i0 + r - 1}]"
            check_output(tag + ".o", got["o"][0, h, i0:i0 + r], o[0, 0], F16)
            check_lse(tag + ".lse", got["lse"][0, h, i0:i0 + r], lse[0, 0], F16)
            check_grad(tag + ".dq1", got["dq1"][0, h, i0:i0 + r], dq1[0, 0], F16)
            check_grad(tag + ".dq2", got["dq2"][0, h, i0:i0 + r], dq2[0, 0], F16)
        tail = 64
        rows = [f[n][:, :, S - tail:] if n in ("q1", "q2", "do") else f[n] for n in PW_NAMES]
        _, dk1, _, dk2, dv = oracle.pw_bwd(*rows, True, c, w)
        tag = f"long_pw[h={h}, keys {S - tail}..{S - 1}]"
        check_grad(tag + ".dk1", got["dk1"][0, h, S - tail:], dk1[0, 0, S - tail:], F16)
        check_grad(tag + ".dk2", got["dk2"][0, h, S - tail:], dk2[0, 0, S - tail:], F16)
        check_grad(tag + ".dv", got["dv"][0, h, S - tail:], dv[0, 0, S - tail:], F16)
