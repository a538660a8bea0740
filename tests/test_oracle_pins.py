"""The CPU oracle against its pins (closed forms, hand-worked case, LAPACK,
torch's AdamW, brute force, invariants).  No GPU needed."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_mod):
    pin(oracle_mod)
