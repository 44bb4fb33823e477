"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(oracle)


from oracle import formats as _formats  # noqa: E402
from oracle_pins_formats import PINS_FORMATS  # noqa: E402


@pytest.mark.parametrize("pin", PINS_FORMATS, ids=[p.__name__ for p in PINS_FORMATS])
def test_formats_oracle_pin(pin):
    pin(_formats)
