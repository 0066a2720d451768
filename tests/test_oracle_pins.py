"""The oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(orc, name):
    assert orc.mutation() == 0
    oracle_pins.ALL_PINS[name](orc)
