"""The oracle against what the pages and the mathematics fix (no GPU)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=[p.__name__ for p in oracle_pins.PINS])
def test_pin(pin, oracle_lib):
    pin(oracle_lib)
