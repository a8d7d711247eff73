"""The CPU oracle against the pages' worked example, library routines, closed forms
and invariants (see oracle_pins.py for what each pin fixes)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)
