"""The oracle's quantizer against its pins (CPU only)."""
import pytest

import quant_pins


@pytest.mark.parametrize("pin", quant_pins.ALL_QPINS, ids=lambda p: p.__name__)
def test_quantizer_pin(orc, pin):
    pin(orc)
