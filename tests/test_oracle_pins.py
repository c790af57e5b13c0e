"""The oracle against its pins (format definition, PyTorch codecs and SDPA,
closed forms, invariants).  CPU only."""

import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
