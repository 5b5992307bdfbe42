"""The CPU oracle against its pins (hand-worked values, closed forms, numpy's
IEEE half conversion, exact rational brute force).  CPU only."""
import numpy as np
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


@pytest.mark.parametrize("call", [
    lambda o: o.pack(np.zeros((12, 8), np.uint8)),                           # K not 8-aligned
    lambda o: o.pack_zeros(np.zeros((1, 20), np.uint8)),                     # N not 8-aligned
    lambda o: o.dequant(np.zeros((1, 16), np.int32), np.zeros((2, 16), np.uint16), None, 8),
    lambda o: o.linear(np.zeros((1, 16), np.uint16), np.zeros((2, 16), np.int32),
                       np.zeros((2, 16), np.uint16), np.zeros((2, 3), np.int32), 8),
    lambda o: o.linear(np.zeros((1, 8), np.uint16), np.zeros((2, 16), np.int32),
                       np.zeros((2, 16), np.uint16), None, 8),                # K mismatch
    lambda o: o.quantize(np.zeros((24, 8), np.uint16), 16, False),
])
def test_oracle_rejects_shapes_the_layout_cannot_hold(oracle_lib, call):
    """Shapes the packed layout cannot hold raise before the C code touches memory."""
    with pytest.raises(ValueError):
        call(oracle_lib)
