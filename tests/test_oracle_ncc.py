"""The NCC oracle against its pins (CPU only)."""
import pytest

import pins_ncc


@pytest.mark.parametrize("pin", pins_ncc.ALL_PINS, ids=lambda f: f.__name__)
def test_ncc_oracle_pin(pin):
    pin()


def test_ncc_oracle_rejects_u32_overflow():
    """A template larger than 66,051 pixels over a saturated image would wrap a
    32-bit SumISq; the oracle reports it instead of returning wrapped sums."""
    import numpy as np
    import oracle

    img = np.full((2, 33040), 255, dtype=np.uint8)  # 2 x 33040 = 66,080 > 66,051
    tmpl = np.full((2, 33040), 255, dtype=np.uint8)
    with pytest.raises(OverflowError):
        oracle.ncc_u8(img, 33040, 2, tmpl)
    ok = np.full((1, 66048), 255, dtype=np.uint8)  # 66,048 <= 66,051: fits
    r = oracle.ncc_u8(ok, 66048, 1, ok)
    assert int(r["sum_isq"][0, 0]) == 65025 * 66048
