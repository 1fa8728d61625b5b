"""The CPU oracle against its pins (closed forms, invariants, page facts,
brute force).  Runs without a GPU."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
