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


def test_sr_random_operand_by_24_bit_multiply_add():
    """The SR encoder forms ~(w << 16), the random operand of an even
    element, with one v_mad_i32_i24: the signed 24-bit low part of w times
    -2^16, minus 1, modulo 2^32.  The low 32 bits of that product depend only
    on the low 16 bits of w, so the identity holds for every w; checked on
    all 2^16 low halves under several high halves (sign bit of the 24-bit
    field set and clear)."""
    import numpy as np
    lo = np.arange(1 << 16, dtype=np.int64)
    for hi in (0x0000, 0x007F, 0x0080, 0x00FF, 0x1234, 0xFF80, 0xFFFF):
        w = (hi << 16) | lo
        a = w & 0xFFFFFF
        a = np.where(a >= 1 << 23, a - (1 << 24), a)  # sign-extend the 24-bit field
        mad = (a * -65536 - 1) & 0xFFFFFFFF
        want = ~(w << 16) & 0xFFFFFFFF
        assert np.array_equal(mad, want), hex(hi)
