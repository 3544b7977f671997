"""The float64 oracle against brute force, closed forms, invariants and the
hand-derived fixtures (CPU only)."""

import pytest

from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()
