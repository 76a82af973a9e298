"""Writes tests/golden/oracle_regression.json from the fp64 oracle only.

The fixture freezes the oracle's outputs on small seeded inputs so that any
later change to the oracle's arithmetic shows up as a failing test and has to
be justified by the passage of the pages it follows.  Run from the repo root:
    python tests/golden/make_golden.py
"""

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")


def inputs(seed):
    rng = np.random.default_rng(seed)
    return {n: rng.standard_normal((1, 2, 8, 4)) for n in ("q", "k", "v", "do", "tq", "tk", "tv", "q2", "k2")}


def cases():
    t = inputs(2024)
    out = {}
    for causal in (False, True):
        c = 0.6
        o, lse = oracle.attn_fwd(t["q"], t["k"], t["v"], causal, c)
        dq, dk, dv = oracle.attn_bwd(t["q"], t["k"], t["v"], t["do"], causal, c)
        _, _, to, _ = oracle.attn_fwd_jvp(t["q"], t["k"], t["v"], t["tq"], t["tk"], t["tv"], causal, c)
        po, plse = oracle.pw_fwd(t["q"], t["k"], t["q2"], t["k2"], t["v"], causal, c, 2)
        pg = oracle.pw_bwd(t["q"], t["k"], t["q2"], t["k2"], t["v"], t["do"], causal, c, 2)
        tag = "causal" if causal else "full"
        out[f"attn_{tag}"] = {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv, "to": to}
        out[f"pw_{tag}"] = {"o": po, "lse": plse, "dq1": pg[0], "dk1": pg[1], "dq2": pg[2],
                            "dk2": pg[3], "dv": pg[4]}
    rng = np.random.default_rng(77)
    x, y0, gy = (rng.standard_normal((6, 16)) for _ in range(3))
    q = rng.standard_normal(16) / 4
    l0, gl = rng.standard_normal(6), rng.standard_normal(6)
    y, lse = oracle.merge_fwd(x, q, y0, l0, 1e-6)
    gx, gq, gy0, gl0 = oracle.merge_bwd(x, q, y0, l0, gy, gl, 1e-6)
    out["merge"] = {"y": y, "lse": lse, "gx": gx, "gq": gq, "gy0": gy0, "gl0": gl0}
    return out


def main():
    data = {k: {n: np.asarray(a).ravel().tolist() for n, a in v.items()} for k, v in cases().items()}
    with open(OUT, "w") as f:
        json.dump({"generator": "tests/golden/make_golden.py (oracle only)", "cases": data}, f)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
