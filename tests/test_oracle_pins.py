"""The CPU oracle against values the pages and mathematics fix (see oracle_pins)."""

import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
