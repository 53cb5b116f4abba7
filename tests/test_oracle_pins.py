"""The fp64 oracle against its pins (closed forms, invariants, one-hot cases,
a 40-digit decimal evaluation); see ``oracle_pins.py`` for what each fixes."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    if not __import__("os").path.exists(oracle.LIB_PATH):
        oracle.build()
    return oracle.LIB_PATH


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
