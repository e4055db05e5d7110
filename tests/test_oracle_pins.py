"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL, ids=[p.__name__ for p in pins.ALL])
def test_pin(o, pin):
    pin(o)
