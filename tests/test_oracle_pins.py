"""The CPU oracle against what the pages and the mathematics fix."""
import os

import pytest

from pins import ALL_PINS

# The sanitizer check (tests/test_sanitizers.py) runs every pin in its quick
# form on an ASan/UBSan build of the oracle.
QUICK = os.environ.get("PINS_QUICK") == "1"


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc, quick=QUICK)
