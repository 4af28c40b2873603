"""The fp64 oracle against facts fixed by the pages and by mathematics
(brute force, closed forms, invariants, hand-worked golden cases)."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
