"""The CPU oracle against its pins (closed forms, invariants, library routines,
high-precision brute force).  See tests/pins.py for what each check fixes."""
import pytest

from pins import PINS


@pytest.mark.parametrize("check", PINS, ids=[c.__name__ for c in PINS])
def test_oracle_pin(orc, check):
    check(orc)
