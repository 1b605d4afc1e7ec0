"""The CPU oracle against what the mathematics fixes (runs without a GPU)."""
import pytest

import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)


def test_oracle_uses_threads(oracle):
    assert oracle.num_threads() >= 1
