"""The oracle's epilogues against their pins (CPU only)."""
import pytest

import epilogue_pins


@pytest.mark.parametrize("pin", epilogue_pins.ALL_EPINS, ids=lambda p: p.__name__)
def test_epilogue_pin(orc, pin):
    pin(orc)
