"""The oracle still reproduces its committed snapshot (tests/golden)."""

import json
import os

import numpy as np

from tests.golden.make_golden import HERE, compute


def test_oracle_matches_snapshot():
    with open(os.path.join(HERE, "oracle_snapshot.json")) as f:
        ref = json.load(f)
    now = compute()
    assert now["codes"] == ref["codes"]
    assert now["packed"] == ref["packed"]
    assert now["zeros"] == ref["zeros"]
    assert np.allclose(now["scales"], ref["scales"], rtol=1e-12)
    assert np.allclose(now["H_diag"], ref["H_diag"], rtol=1e-12)
    assert np.allclose(now["U_diag"], ref["U_diag"], rtol=1e-10)
    assert abs(now["loss"] - ref["loss"]) <= 1e-10 * abs(ref["loss"])
