"""The CPU oracle against its pins (library routines, closed forms, golden
fixtures, invariants, and the independent brute-force twin)."""
import pytest

from tests.oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(orc, name):
    PINS[name](orc)
