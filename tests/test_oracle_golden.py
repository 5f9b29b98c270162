"""The oracle's outputs on small seeded workloads match the stored digests
written by tests/golden/make_golden.py (a guard against unintended changes to
the oracle's arithmetic or to the input recipes)."""
import json
import os
import sys

HERE = os.path.dirname(__file__)
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_oracle_digests_unchanged():
    stored = json.load(open(os.path.join(HERE, "golden", "oracle_digests.json")))
    stored.pop("_source")
    assert make_golden.compute() == stored
