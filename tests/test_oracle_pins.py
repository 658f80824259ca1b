"""The CPU oracle checked against its pins (closed forms, mpmath, the page's block
matrix R, complex multiplication, invariants, exact rationals, brute force)."""
import pytest

import oracle
from oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=[c.__name__ for c in ALL_CHECKS])
def test_oracle_pin(check):
    check(oracle.default())
