"""The oracle still reproduces its committed tiny-workload fixture."""

import json
import os

from tests.golden.make_golden import compute


def test_tiny_fixture_unchanged():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_decode_1x1k_seed1.json")
    with open(path) as f:
        want = json.load(f)
    assert compute() == want
