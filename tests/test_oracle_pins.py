"""The CPU oracle against what the pages and the mathematics fix (tests/pins.py)."""
import pytest

import pins
from oracle import ssu_oracle


@pytest.fixture(scope="module")
def orc():
    return ssu_oracle.default()


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
