"""CPU pins of the fp64 oracle (see oracle_pins.py for what each check compares against)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.Oracle()


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(o, check):
    check(o)
