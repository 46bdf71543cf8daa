"""The CPU oracle against what the pages and the mathematics fix (runs without a GPU)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(name):
    ALL_PINS[name]()
