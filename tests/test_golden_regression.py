"""The oracle's results on the tiny workload must not drift: digests written by
tests/golden/make_golden.py (which calls only the oracle)."""
import json
import os

import pytest

from tests.golden import make_golden

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")))


def test_oracle_tiny_workload_is_stable():
    now = make_golden.compute()
    for key, val in GOLD.items():
        if isinstance(val, float):
            assert now[key] == pytest.approx(val, rel=1e-12), key
        elif isinstance(val, list):
            assert now[key] == pytest.approx(val, rel=1e-12), key
        else:
            assert now[key] == val, key
