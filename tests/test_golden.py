"""The oracle still reproduces its committed regression fixture (written from oracle/ only)."""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.join(os.path.dirname(__file__), "golden"))
import make_golden  # noqa: E402


def test_oracle_matches_fixture():
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")
    want = json.load(open(path))
    got = make_golden.build()
    assert np.allclose(got["probs"], want["probs"], rtol=1e-12, atol=1e-15)
    assert got["mask"] == want["mask"]
    assert np.allclose(got["kept_mass"], want["kept_mass"], rtol=1e-12)
    assert np.allclose(got["out_rows"], want["out_rows"], rtol=1e-11, atol=1e-12)
