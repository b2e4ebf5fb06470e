"""The CPU oracle against its pins (hand-worked values, exact arithmetic,
closed forms, the pages' printed sizes). CPU only."""

import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, pin):
    pin(oracle_mod)
