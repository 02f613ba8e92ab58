"""Each planted mistake in the oracle (a dropped or sign-flipped minimum, the
wrong nibble order, the wrong group size, a transposed scale read, a dropped
term of the sum, a wrong activation row; in the quantizer a lost top code,
truncation for rounding, 16 steps for 15; in the epilogues a sign error in
silu, swapped gate/up halves, a sum for the mean, a dropped eps) must trip
at least two pins.  The
mutants are separate builds of the same C source; CPU only."""
import os
import shutil

import pytest

import oracle
import oracle_pins
import quant_pins
import epilogue_pins
from oracle.build import build_oracle

PLANTS = {1: "minimum dropped", 2: "minimum subtracted", 3: "high nibble first",
          4: "groups of 64", 5: "scale read transposed", 6: "last k dropped",
          7: "every row reads x row 0", 8: "quantizer loses code 15", 9: "quantizer truncates",
          10: "quantizer uses 16 steps", 11: "silu with exp(+g)", 12: "gate and up halves swapped",
          13: "rmsnorm sum for mean", 14: "rmsnorm eps dropped"}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p].replace(" ", "_"))
def test_planted_mistake_is_caught(tmp_path, plant):
    lib = build_oracle(out=os.path.join(str(tmp_path), f"mutant{plant}.so"), plant=plant)
    mutant = oracle.Oracle(lib)
    assert mutant.plant == plant
    caught = []
    for pin in oracle_pins.ALL_PINS + quant_pins.ALL_QPINS + epilogue_pins.ALL_EPINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError):
            caught.append(pin.__name__)
    assert len(caught) >= 2, f"planted mistake {plant} ({PLANTS[plant]}) caught only by {caught}"
