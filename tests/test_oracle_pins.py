"""The oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=[p.__name__ for p in pins.ALL])
def test_pin(oracle_lib, pin):
    pin()
