"""Regression pin: SHA-256 of the oracle's outputs on the seeded inputs, recorded by
tests/golden/make_golden.py (which calls only the oracle and the input generator).
The input hashes pin the generator; the output hashes catch any later drift in the
oracle's arithmetic."""
import json
import os

from tests.golden import make_golden


def test_oracle_hashes_unchanged(orc):
    with open(make_golden.OUT) as f:
        want = json.load(f)
    got = make_golden.compute()
    assert got == want
