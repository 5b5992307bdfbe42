"""The CPU oracle against its pins (hand-worked values, closed forms, numpy's
IEEE half conversion, exact rational brute force).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)
