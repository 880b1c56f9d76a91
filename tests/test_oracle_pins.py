"""The fp64 oracle against facts fixed by the definition of softmax attention."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_pin(lib, name):
    oracle_pins.ALL_PINS[name](lib)
