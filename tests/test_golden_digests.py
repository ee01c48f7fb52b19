"""The seeded generators and the CPU oracle still produce the stored digests
(tests/golden/oracle_digests.json, written by tests/golden/make_golden.py)."""
import json
import os

import pytest

from tests.golden.make_golden import CASES, case_digests

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("name,scale_down", CASES)
def test_digests_unchanged(name, scale_down):
    with open(os.path.join(HERE, "golden", "oracle_digests.json")) as f:
        stored = json.load(f)[f"{name}/{scale_down or 1}"]
    got = case_digests(name, scale_down)
    assert got["inputs"] == stored["inputs"]
    assert got["lists"] == stored["lists"]
    assert got["scores_f32"] == stored["scores_f32"]
