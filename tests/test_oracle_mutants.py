"""Every planted mistake in the oracle fails at least one pin (CPU only).

The mistakes are compiled into separate copies of oracle.c with
ORACLE_MUTANT=k; the real oracle is never modified.  The list (see the
mutant switches in oracle.c): square in double, float accumulator, last
column dropped, stride ignored, ref/dis swapped, PSNR rows reversed, PSNR
terms added straight into the frame sum, first moment halved, noise square
in double, MSE divided by the width, scaler off by one bit, a batch's
frame pitch taken as bytes, a batch's frames assumed packed, the dB peak
of 8-bit samples at every depth.
"""
import os

import pytest

import oracle
import oracle_checks

MUTANTS = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 13, 14, 15]


@pytest.mark.parametrize("mutant", MUTANTS)
def test_mutant_is_caught(tmp_path, mutant):
    so = oracle.build(out=os.path.join(tmp_path, f"liboracle_m{mutant}.so"),
                      mutant=mutant)
    orc = oracle.Oracle(oracle.load(so))
    caught = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check(orc)
        except AssertionError:
            caught.append(check.__name__)
    assert caught, f"mutant {mutant} passed every pin"
