"""Each plausible mistake planted in a copy of the oracle source must fail at least one pin."""
import pytest

import pins
from mutants import MUTANTS, build_mutant


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    orc = build_mutant(name, str(tmp_path))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
