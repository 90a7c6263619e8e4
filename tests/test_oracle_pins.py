"""The fp64 oracle against closed forms, a library routine and invariants (CPU)."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin, oracle_lib):
    pin(oracle_lib)
