"""The CPU oracle against its pins (library routines, closed forms, invariants, fixtures)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(orc, name):
    ALL_PINS[name](orc)
