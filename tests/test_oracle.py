"""The fp64 oracle against its pins (hand-worked fixtures, exact rational
brute force, closed forms, linearity, row independence).  CPU only."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    assert orc.plant == 0
    pin(orc)


def test_rejects_bad_shapes(orc):
    import numpy as np
    import oracle
    W = np.zeros((2, 16), dtype=np.uint32)
    s = np.zeros((2, 1), dtype=np.uint16)
    with pytest.raises(oracle.OracleError):
        orc.gemm(np.zeros((1, 64), dtype=np.uint16), W, s, s)
    with pytest.raises(oracle.OracleError):
        orc.dequant_f64(W, np.zeros((2, 2), dtype=np.uint16), s)


def test_rejects_nonfinite(orc):
    import numpy as np
    import oracle
    W = np.zeros((1, 16), dtype=np.uint32)
    s = np.full((1, 1), 0x7F80, dtype=np.uint16)   # +inf
    with pytest.raises(oracle.OracleError):
        orc.dequant_f64(W, s, s)


def test_thread_count_does_not_change_results(orc):
    import numpy as np
    import synth
    case = synth.make_random(2, 1024, 37, 61)
    wt = case.weights
    y1, a1 = orc.gemm(case.x, wt.W, wt.scale, wt.mn, nthreads=1)
    y4, a4 = orc.gemm(case.x, wt.W, wt.scale, wt.mn, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(a1, a4)
