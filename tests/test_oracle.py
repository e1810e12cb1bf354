"""The fp64 oracle against its pins (CPU only).  See tests/oracle_pins.py."""
import pytest

import oracle_pins
from oracle import oracle as orc


@pytest.fixture(scope="module")
def lib():
    orc.build(force=False)
    return orc.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
