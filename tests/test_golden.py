"""The generator's byte stream and the oracle's values for the small
single-GEMV workload (Q4_K/Q5_K/Q6_K, 256 x 2560, batch 1) match the record
written by tests/golden/make_golden.py (self-generated: the K-quant kernel
arc page prints no worked values)."""
import json
import os

import pytest

from golden.make_golden import record

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def stored():
    with open(os.path.join(HERE, "golden", "c0_oracle.json")) as f:
        return json.load(f)


def test_generator_and_oracle_match_stored_record(stored):
    assert record() == stored
