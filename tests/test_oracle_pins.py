"""The CPU oracle against its pins (hand-worked golden cases, closed forms,
invariants and independent library routines)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](oracle.lib())
