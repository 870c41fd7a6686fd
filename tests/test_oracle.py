"""The oracle against its pins (CPU only)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("pin", oracle_pins.HELPER_PINS, ids=lambda f: f.__name__)
def test_helper_pin(pin):
    import oracle
    pin(oracle)
