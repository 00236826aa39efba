"""The fp64 oracle against library routines, closed forms, the band fixture and invariances."""
import pytest

from oracle import oracle as oracle_mod
from tests import pins


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
