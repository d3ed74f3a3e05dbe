"""The fp64 oracle against what the mathematics fixes (CPU only)."""
import pytest

import oracle_pins
from oracle import default


@pytest.fixture(scope="module")
def ref():
    return default()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(ref, pin):
    pin(ref)
