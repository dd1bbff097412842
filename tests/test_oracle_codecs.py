"""Pins of the oracle's format codecs against things other than itself.

* E2M1 decode against the bit-field definition of the OCP FP4 format
  (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).
* E4M3 decode against torch's float8_e4m3fn, exhaustively (256 bytes).
* E4M3 encode against torch's float32 -> float8_e4m3fn cast (round to nearest
  even), exhaustively over several whole binades and on every midpoint +-1ulp.
* E2M1 round-to-nearest-even against an independent encoder built on
  numpy.rint (round half to even), exhaustively over every fp32 bit pattern
  with 2^-4 <= |y| < 8 and on samples outside.
* E2M1 stochastic rounding: support {lo, hi}, exact threshold, and the worked
  example of "Pretraining Large Language Models with NVFP4" (lay part, "De
  Vier Slimme Trucs", the rounding of 3.4): P(3) = 0.6, P(4) = 0.4.
* Dequantize: every (code, scale byte) pair under five tensor scales against
  the bit-field E2M1 value times torch's E4M3 value, divided once in double.
"""
import json
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_from_bits(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


# ---------------------------------------------------------------- E2M1 ---
def e2m1_from_fields(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    v = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
    return -v if s else v


def test_e2m1_decode_matches_bit_fields(orc):
    for code in range(16):
        want = e2m1_from_fields(code)
        got = orc.e2m1_value(code)
        assert got == want and np.signbit(got) == np.signbit(want), code
    mags = sorted({abs(orc.e2m1_value(c)) for c in range(16)})
    assert mags == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def rne_reference(y):
    """Independent E2M1 RNE: round to the grid's local step with np.rint."""
    y = np.asarray(y, dtype=np.float32)
    m = np.abs(y.astype(np.float64))
    q = np.where(m < 2, np.rint(m * 2) / 2, np.where(m < 4, np.rint(m), np.rint(m / 2) * 2))
    q = np.minimum(q, 6.0)
    lut = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    idx = np.zeros(q.shape, dtype=np.uint8)
    for v, i in lut.items():
        idx[q == v] = i
    return (np.signbit(y).astype(np.uint8) << 3) | idx


def test_e2m1_rne_tie_table(orc):
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for y, idx in ties.items():
        assert orc.e2m1_encode_rne(y) == idx
        assert orc.e2m1_encode_rne(-y) == 8 | idx
    assert orc.e2m1_encode_rne(0.0) == 0
    assert orc.e2m1_encode_rne(-0.0) == 8
    assert orc.e2m1_encode_rne(-1e-30) == 8
    assert orc.e2m1_encode_rne(6.0) == 7
    assert orc.e2m1_encode_rne(1e30) == 7
    assert orc.e2m1_encode_rne(float("inf")) == 7
    assert orc.e2m1_encode_rne(float("-inf")) == 15


def test_e2m1_rne_exhaustive_core_range(orc):
    # every fp32 pattern with exponent field 123..129 (2^-4 <= |y| < 8), both signs
    lo = np.uint32(123 << 23)
    hi = np.uint32(130 << 23)
    bits = np.arange(lo, hi, dtype=np.uint32)
    for sign in (0, 0x80000000):
        y = f32_from_bits(bits | np.uint32(sign))
        for chunk in np.array_split(np.arange(y.size), 8):
            got = orc.e2m1_encode_rne_n(y[chunk])
            want = rne_reference(y[chunk])
            bad = np.nonzero(got != want)[0]
            assert bad.size == 0, (y[chunk][bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_rne_samples_outside(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    y = f32_from_bits(bits)
    y = y[np.isfinite(y)]
    got = orc.e2m1_encode_rne_n(y)
    want = rne_reference(y)
    assert np.array_equal(got, want)


def test_e2m1_sr_support_and_threshold(orc):
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    rng = np.random.default_rng(2)
    y = rng.uniform(-6.5, 6.5, size=200_000).astype(np.float32)
    u = rng.integers(0, 65536, size=y.size).astype(np.uint16)
    codes = orc.e2m1_encode_sr_n(y, u)
    vals = np.array([orc.e2m1_value(c) for c in range(16)])[codes]
    m = np.abs(y.astype(np.float64))
    g = np.array(grid)
    lo_idx = np.clip(np.searchsorted(g, m, side="right") - 1, 0, 7)
    lo = g[lo_idx]
    hi = g[np.minimum(lo_idx + 1, 7)]
    # support: always one of the two neighbours (6 when saturated)
    ok = (np.abs(vals) == lo) | (np.abs(vals) == hi)
    assert ok.all()
    # threshold: up iff u < f * 2^16 (f exact), checked against integer form
    inside = m < 6
    f = (m - lo) / np.where(hi > lo, hi - lo, 1)
    up = u.astype(np.float64) < f * 65536
    assert np.array_equal((np.abs(vals) == hi)[inside & (hi > lo)], up[inside & (hi > lo)])
    # sign is kept
    assert np.array_equal(codes >> 3, np.signbit(y).astype(np.uint8))


def test_e2m1_sr_grid_points_exact(orc):
    for v in [0, 0.5, 1, 1.5, 2, 3, 4, 6]:
        for u in (0, 1, 32767, 65535):
            assert abs(orc.e2m1_value(orc.e2m1_encode_sr(v, u))) == v


def test_sr_worked_example_from_pages(orc):
    """3.4 rounds to 3 with probability 0.6 and to 4 with probability 0.4."""
    with open(os.path.join(GOLDEN, "sr_worked_example.json")) as f:
        ex = json.load(f)
    x = np.float32(ex["x"])
    n = 1 << 20
    u = orc.sr_bits_n(seed=0, stream=0, first=0, n=n)
    codes = orc.e2m1_encode_sr_n(np.full(n, x, dtype=np.float32), u)
    vals = np.array([orc.e2m1_value(c) for c in range(16)])[codes]
    assert set(np.unique(vals)) <= {ex["lo"], ex["hi"]}
    p_hi = np.mean(vals == ex["hi"])
    sigma = np.sqrt(ex["p_hi"] * (1 - ex["p_hi"]) / n)
    assert abs(p_hi - ex["p_hi"]) < 5 * sigma
    # the page's contrast: always rounding down 100 times loses about 40 in total
    assert abs(ex["n"] * (float(x) - ex["lo"]) - ex["always_down_error"]) < 1e-3


# ---------------------------------------------------------------- E4M3 ---
def test_e4m3_decode_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        got = orc.e4m3_value(b)
        if np.isnan(t[b]):
            assert np.isnan(got), b
        else:
            assert got == t[b] and np.signbit(got) == np.signbit(t[b]), b
    assert orc.e4m3_value(0x7E) == 448.0
    assert orc.e4m3_value(0x01) == 2.0 ** -9
    assert orc.e4m3_value(0x08) == 2.0 ** -6
    assert orc.e4m3_value(0x38) == 1.0


def torch_e4m3(s):
    return torch.from_numpy(np.ascontiguousarray(s)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_whole_binades(orc):
    # every fp32 in [2^-12, 2^-7) (subnormal/normal boundary of E4M3) and in
    # [128, 464] (top of the range, incl. the tie at 464 -> 448)
    for lo_e, hi_e in ((115, 120), (134, 136)):
        bits = np.arange(np.uint32(lo_e << 23), np.uint32(hi_e << 23), dtype=np.uint32)
        s = f32_from_bits(bits)
        s = s[s <= 464.0]
        assert np.array_equal(orc.e4m3_encode_n(s), torch_e4m3(s))


def test_e4m3_encode_midpoints(orc):
    vals = np.array([orc.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    cand = [mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf), vals.astype(np.float32)]
    s = np.concatenate(cand)
    s = s[(s >= 0) & (s <= 464)]
    assert np.array_equal(orc.e4m3_encode_n(s), torch_e4m3(s))
    # ties resolve to the even byte, e.g. 2^-10 (between 0 and 2^-9) -> 0
    assert orc.e4m3_encode(2.0 ** -10) == 0
    assert orc.e4m3_encode(448.0 * 1.01) == 0x7E
    assert orc.e4m3_encode(float("inf")) == 0x7E


def test_e4m3_encode_random(orc):
    rng = np.random.default_rng(3)
    s = np.exp(rng.uniform(np.log(1e-45), np.log(464), size=3_000_000)).astype(np.float32)
    s = s[s <= 464]
    assert np.array_equal(orc.e4m3_encode_n(s), torch_e4m3(s))


# ---------------------------------------------------------- dequantize ---
@pytest.mark.parametrize("s_enc", [1.0, 2688.0 / 3.7, 3.4028234663852886e38, 7.899e-36, 0.3])
def test_dequantize_every_code_and_scale_byte(orc, s_enc):
    # "Pretraining Large Language Models with NVFP4", 2A: an element is its
    # E2M1 code times its block's E4M3 scale, over the FP32 tensor scale.
    # Independent route: E2M1 from its bit fields, E4M3 through torch's
    # float8_e4m3fn, one correctly rounded division in double (the product of
    # a 2-bit and a 4-bit significand is exact, so there is one rounding).
    # Row r holds one block: codes 0 .. 15 under scale byte r (0x00 .. 0x7E).
    s32 = float(np.float32(s_enc))
    codes = np.tile(np.array([(2 * k) | ((2 * k + 1) << 4) for k in range(8)], np.uint8), (127, 1))
    scales = np.arange(127, dtype=np.uint8).reshape(127, 1)
    got = orc.dequantize(codes, scales, s32)
    e4m3 = torch.from_numpy(scales.ravel().copy()).view(torch.float8_e4m3fn).double().numpy()
    e2m1 = np.array([e2m1_from_fields(c) for c in range(16)], np.float64)
    want = (e2m1[None, :] * e4m3[:, None]) / s32
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got[:, 8]), np.ones(127, bool))  # code 8 is -0
