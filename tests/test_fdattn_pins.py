"""The flash deformable attention oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import fdattn_pins


@pytest.fixture(scope="session")
def fdattn_lib():
    return oracle.load_fdattn()


@pytest.mark.parametrize("pin", fdattn_pins.PINS, ids=lambda f: f.__name__)
def test_pin(pin, fdattn_lib):
    pin(fdattn_lib)
