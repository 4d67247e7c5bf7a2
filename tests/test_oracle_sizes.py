"""Pins for the oracle's row and fixed-slot buffer sizing against the byte
counts the pages print (tests/golden/page_sizes.json, each case cited)."""
import json
import os

import pytest

import oracle

_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")
CASES = json.load(open(_GOLDEN))["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["what"][:40] for c in CASES])
def test_printed_sizes(case):
    dtype = oracle.BF16 if case["dtype"] == "bf16" else oracle.FP8_E4M3
    got = oracle.fixed_slot_bytes(case["experts"], case["slots"], case["H"], dtype, case["header"])
    val = got / case["unit_bytes"]
    if case["rounding"] == "exact":
        assert val == case["printed"]
    elif case["rounding"] == "nearest":
        assert round(val) == case["printed"]
    elif case["rounding"] == "one_decimal":
        assert round(val, 1) == case["printed"]
    else:
        raise AssertionError(case["rounding"])


def test_row_bytes_match_layout():
    assert oracle.row_bytes(4096, oracle.BF16) == 8192
    assert oracle.row_bytes(6144, oracle.FP8_E4M3) == 6144 + 48 * 4
