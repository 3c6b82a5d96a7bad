"""Run every oracle pin (tests/oracle_pins.py) on the oracle built from oracle/arrms_oracle.c."""
import pytest

import oracle
from tests.oracle_pins import PINS


@pytest.mark.parametrize("name,fn,kw", PINS, ids=[p[0] for p in PINS])
def test_oracle_pin(name, fn, kw):
    fn(oracle.default(), **kw)
