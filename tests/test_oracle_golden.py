"""The oracle still reproduces the frozen fixture written by
tests/golden/make_golden.py (a script that calls only the oracle)."""

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_matches_frozen_fixture():
    with open(os.path.join(HERE, "golden", "oracle_regression.json")) as f:
        frozen = json.load(f)["cases"]
    now = make_golden.cases()
    assert set(frozen) == set(now)
    for case, arrs in now.items():
        for name, a in arrs.items():
            np.testing.assert_allclose(np.asarray(a).ravel(), np.asarray(frozen[case][name]),
                                       atol=1e-12, rtol=0, err_msg=f"{case}.{name}")
