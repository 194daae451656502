"""The oracle against its frozen regression fixture (CPU only)."""

import json
import os

import numpy as np

from golden import make_golden


def test_oracle_matches_frozen_fixture():
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")
    with open(path) as f:
        want = json.load(f)
    got = make_golden.build()
    assert sorted(got) == sorted(want)
    for case in want:
        for key in want[case]:
            a = np.asarray(got[case][key], dtype=np.float64)
            b = np.asarray(want[case][key], dtype=np.float64)
            assert np.allclose(a, b, rtol=1e-12, atol=1e-12), (case, key)
