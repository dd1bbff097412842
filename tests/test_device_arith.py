"""Host checks of arithmetic identities that the device encoder relies on.

These are not oracle pins: the oracle divides by 6 with one IEEE division.
They show that the device's cheaper form gives the same scale bytes, which
the GPU parity tests then confirm end to end.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(__file__)


@pytest.mark.slow
def test_div6_correction_is_exact(tmp_path):
    exe = str(tmp_path / "div6_check")
    # -ffp-contract=off: the product t * c must stay a separate rounding
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "helpers", "div6_check.c"), "-lm"], check=True)
    normal, tiny = map(int, subprocess.run([exe], capture_output=True, text=True,
                                           check=True).stdout.split())
    # correctly rounded for every t in [2^-125, FLT_MAX]
    assert normal == 0
    # below 2^-125 the quotient (< 2^-127) encodes to the zero E4M3 byte
    # whichever way its last subnormal bit goes; the count documents that
    # the correction is not exact there
    assert tiny > 0
