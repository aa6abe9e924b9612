"""The oracle against its pins: hand-worked fixtures, closed forms, brute
force, library routines and invariants (all on the CPU)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
