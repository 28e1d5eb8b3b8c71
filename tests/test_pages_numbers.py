"""The pages' printed figures are quoted consistently (tests/golden/pages_numbers.json)."""

import json
import os

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_pages_derived_ratios():
    g = json.load(open(os.path.join(GOLD, "pages_numbers.json")))
    for r in g["ratios"]:
        got = r["num"] / r["den"]
        assert abs(got - r["printed"]) <= r["tol"], r
