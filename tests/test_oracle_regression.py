"""The oracle's outputs on small seeded inputs stay what the committed fixture says."""
import json
import os

import numpy as np

from tests.golden.make_golden import compute


def test_oracle_matches_frozen_outputs():
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")) as f:
        frozen = json.load(f)
    now = compute()
    assert len(now) == len(frozen)
    for a, b in zip(now, frozen):
        for key in b:
            assert np.array_equal(np.asarray(a[key]), np.asarray(b[key])), key
