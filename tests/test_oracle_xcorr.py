"""The cross-correlation oracle against its pins (CPU only)."""
import pytest

import pins_xcorr


@pytest.mark.parametrize("pin", pins_xcorr.ALL_PINS, ids=lambda f: f.__name__)
def test_xcorr_oracle_pin(pin):
    pin()
