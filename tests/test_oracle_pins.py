"""The oracle against its pins (closed forms, invariants, library special
cases, brute force) -- CPU only."""
import pytest

import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle, pin):
    pin(oracle)
