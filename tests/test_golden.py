"""The oracle still reproduces its frozen tiny-layer fixture (regression
guard on the oracle's arithmetic; see tests/golden/README.md)."""
import json
import os

import numpy as np

from tests_golden_loader import load_builder

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_frozen_fixture():
    ref = json.load(open(os.path.join(HERE, "golden", "oracle_tiny_layer.json")))
    now = load_builder()()
    for key in ("ids", "counts", "offsets", "sorted_assign", "assign_pos"):
        assert now[key] == ref[key], key
    assert np.allclose(now["gates"], ref["gates"], rtol=0, atol=0)
    assert np.allclose(now["y"], ref["y"], rtol=1e-13, atol=1e-15)
