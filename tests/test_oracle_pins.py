"""The oracle against its pins (values printed on the pages, closed forms,
invariants, brute force).  CPU only."""
import pytest

import oracle as O
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(O)
