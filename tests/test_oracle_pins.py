"""The CPU oracle against its pins (hand cases, textbook routines, identities,
invariants, brute force). Runs without a GPU."""
import pytest

import _pins


@pytest.mark.parametrize("check", _pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()


@pytest.mark.parametrize("case", _pins.golden_cases(), ids=lambda c: c["name"])
def test_hand_case(case):
    _pins.check_hand_case(case)
