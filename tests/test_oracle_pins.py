"""The oracle against brute force, closed forms, invariants and the hand-worked example (CPU only)."""

import pytest

from pins_oracle import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name]()
