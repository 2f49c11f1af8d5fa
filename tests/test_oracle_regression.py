"""The oracle's config-0 result is frozen in tests/golden/regression_c0.json (written by make_golden.py)."""
import json
import os

from golden_loader import load_make_golden


def test_oracle_config0_digest_unchanged():
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "regression_c0.json")) as f:
        want = json.load(f)
    assert load_make_golden().compute() == want
