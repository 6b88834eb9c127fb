"""The CPU oracle against its pins (closed forms, library routines, brute
force, the identities and bounds of App. E, a hand-worked example)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_mod):
    pin(oracle_mod)
