"""The oracle reproduces its committed regression fixture (tests/golden/oracle_tiny.json)."""
import json
import os

import numpy as np

from tests.golden.make_oracle_tiny import compute

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_regression_fixture():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as fh:
        ref = json.load(fh)["cases"]
    now = compute()
    for r, c in zip(ref, now):
        for key in ("f", "g", "grad_x"):
            np.testing.assert_allclose(c[key], r[key], rtol=1e-12, atol=1e-14)
        assert abs(c["cost"] - r["cost"]) <= 1e-12 * abs(r["cost"])
