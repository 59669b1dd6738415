"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def ora():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(ora, pin):
    pin(ora)


def test_pin_count():
    # every pin listed in the oracle's documentation is present
    assert len(oracle_pins.ALL_PINS) >= 20
