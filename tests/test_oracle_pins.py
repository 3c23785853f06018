"""The oracle against the pages' printed arithmetic, closed forms, invariants and
a pure-Python brute force (CPU only)."""
import pytest

from tests import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
