"""The oracle against its pins (CPU only).  See oracle_pins.py for what each
check compares the oracle with."""
import pytest

from . import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()
