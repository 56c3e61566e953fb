"""The oracle tower's composition against hand computations
(tests/tower_pins.py): the query/key scaling and relative keys of the
attention, the clamp/SiLU order of the FFN, the norm/SiLU order of the light
conv, and the block order of a layer."""
import pytest

from oracle import tower as tw
from tower_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_tower_pin(pin):
    pin(tw)
