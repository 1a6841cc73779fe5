"""Regression pin: the oracle's output on the tiny workload matches its stored digest.

The digest was written by tests/golden/make_golden.py, which calls only the oracle
and the input generators.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

import make_golden  # noqa: E402


def test_tiny_digest_unchanged():
    with open(os.path.join(HERE, "golden", "tiny_oracle_digest.json")) as f:
        stored = json.load(f)
    assert make_golden.digest() == stored
