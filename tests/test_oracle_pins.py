"""The oracle against its pins (brute force, closed forms, hand examples,
library special cases, invariants). CPU only."""
import pytest

import oracle
from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
