"""The CPU oracle against facts that do not come from it (see tests/oracle_pins.py)."""

import pytest

import oracle
from oracle_pins import CHECKS


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check(oracle._load())
