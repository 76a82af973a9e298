"""GPU parity on one very long head pair: bf16 B1 H2 D128 with 32768 keys
(causal) or 16384 (non-causal).

The forward walks up to 512 key blocks per query block (the running maximum
raised lazily many times over), the dK/dV pass up to 1024 query blocks per
key block, and a head spans 128 (64) query blocks.  The oracle checks exactly
what it can compute in seconds at this length:

* O, LSE and dQ on windows of 8 query rows at the start, the middle and the
  end of each head: a window of rows needs all keys (non-causal) or only the
  keys up to its last row (causal: the oracle's bottom-right alignment of 8
  rows against those keys is the global diagonal);
* causal: dK and dV of the last 64 keys, which only the last 64 query rows
  reach (the oracle's backward over those rows and all keys is exact there);
* every output finite.
"""

import numpy as np
import pytest

import oracle
from attention_fa2_tiles_amd.inputs import BF16, AttnWorkload, attn_inputs
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
