"""Pins of the oracle's MXFP4 functions (OCP Microscaling Formats (MX) v1.0,
section 6.3: a 32-element block shares the scale 2^(floor(log2(amax)) - 2),
stored as an E8M0 byte, and each element is V / scale rounded to E2M1).

Each pin comes from outside the oracle's code: hand-worked examples of the
conversion rule, exact round trips of representable blocks, the scale
exponent re-derived with numpy's frexp, the half-step error bound of
round-to-nearest, and numpy's float64 matmul on an independent
dequantization."""
import numpy as np
import pytest

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def codes_of(packed):
    return np.stack([packed & 15, packed >> 4], -1).reshape(packed.shape[0], -1)


def test_hand_worked_block(orc):
    # amax 7: floor(log2 7) = 2, scale 2^0 (byte 127); 7 saturates to 6,
    # 3.3 -> 3, -0.2 -> -0 (below 0.25), 0.25 -> 0 and 0.75 -> 1 (ties to the
    # even code), 2.5 -> 2 (tie), -5 -> -4 (tie between 4 and 6: even is 4)
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [7.0, 3.3, -0.2, 0.25, 0.75, 2.5, -5.0, 1.4]
    codes, scales = orc.mx_quantize(x)
    assert scales[0, 0] == 127
    want = [7, 5, 8, 0, 2, 4, 8 | 6, 3]   # indices into GRID, sign in bit 3
    assert codes_of(codes)[0, :8].tolist() == want
    assert (codes_of(codes)[0, 8:] == 0).all()
    # amax 0.1: floor(log2 0.1) = -4, scale 2^-6 (byte 121): 0.1 * 64 = 6.4 -> 6
    y = np.zeros((1, 32), np.float32)
    y[0, 0], y[0, 1] = 0.1, -0.03  # -0.03 * 64 = -1.92 -> -2
    codes, scales = orc.mx_quantize(y)
    assert scales[0, 0] == 121
    assert codes_of(codes)[0, :2].tolist() == [7, 8 | 4]


def test_zero_and_tiny_blocks(orc):
    x = np.zeros((2, 64), np.float32)
    x[1, 32] = 8e-39          # amax below 2^-125: the exponent clamps to -127 (byte 0)
    x[1, 33] = -3e-39
    x[1, 34] = 1e-40
    codes, scales = orc.mx_quantize(x)
    assert scales[0].tolist() == [0, 0] and scales[1, 0] == 0 and scales[1, 1] == 0
    # with 2^-127 = 5.877e-39: 8e-39 -> 1.361 -> 1.5; -3e-39 -> -0.510 -> -0.5;
    # 1e-40 -> 0.017 -> 0
    assert codes_of(codes)[1, 32:35].tolist() == [3, 8 | 1, 0]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_representable_blocks_round_trip(orc, dtype):
    rng = np.random.default_rng(0)
    rows, nb = 24, 6
    q = rng.choice(np.concatenate([GRID, -GRID]), size=(rows, nb, 32))
    q[:, :, 0] = rng.choice([4.0, 6.0, -4.0, -6.0], size=(rows, nb))  # pins the block's scale
    e = rng.integers(-20, 20, size=(rows, nb, 1))
    x = (q * 2.0 ** e).reshape(rows, nb * 32).astype(np.float32)
    if dtype == "bf16":
        inp = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: few mantissa bits
    else:
        inp = x
    codes, scales = orc.mx_quantize(inp)
    assert np.array_equal(scales.astype(int) - 127, e[:, :, 0])
    assert np.array_equal(orc.mx_dequantize(codes, scales), x.astype(np.float64))


def test_scale_is_frexp_exponent_and_error_bound(orc):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, size=(64, 1)))).astype(np.float32)
    codes, scales = orc.mx_quantize(x)
    amax = np.abs(x.reshape(64, 8, 32)).max(-1)
    _, e = np.frexp(amax.astype(np.float64))
    assert np.array_equal(scales.astype(int) - 127, e - 1 - 2)
    # round to nearest on the grid: error at most half the local step (the
    # step is 0.5 below 2, 1 in [2, 4), 2 in [4, 6]); above 6 saturation
    deq = orc.mx_dequantize(codes, scales).reshape(64, 8, 32)
    X = 2.0 ** (scales.astype(int) - 127)[:, :, None]
    v = x.reshape(64, 8, 32) / X
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    inside = np.abs(v) <= 6
    err = np.abs(deq / X - v)
    assert (err[inside] <= step[inside] / 2 + 1e-12).all()
    # |V / X| < 8 always; above 6 the code saturates to 6
    assert (np.abs(v) < 8).all()
    assert np.array_equal(np.abs(deq / X)[~inside], np.full((~inside).sum(), 6.0))


def test_dequantize_is_code_times_power_of_two(orc):
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=(8, 32), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(8, 2), dtype=np.uint8)
    vals = np.concatenate([GRID, -GRID])[codes_of(codes)]
    want = vals * 2.0 ** (np.repeat(scales.astype(int), 32, axis=1) - 127)
    assert np.array_equal(orc.mx_dequantize(codes, scales), want)
    assert np.isnan(orc.e8m0_value(0xFF)) and orc.e8m0_value(127) == 1.0 and orc.e8m0_value(0) == 2.0 ** -127


def test_mx_gemm_matches_blas_on_independent_dequant(orc):
    rng = np.random.default_rng(3)
    M, N, K = 40, 24, 160
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = rng.standard_normal((N, K)).astype(np.float32) * 100
    ac, as_ = orc.mx_quantize(a)
    bc, bs = orc.mx_quantize(b)
    grid = np.concatenate([GRID, -GRID])

    def deq(c, s):
        return grid[codes_of(c)] * 2.0 ** (np.repeat(s.astype(int), 32, axis=1) - 127)
    da, db = deq(ac, as_), deq(bc, bs)
    c, absum = orc.mx_gemm(ac, as_, bc, bs)
    assert np.allclose(c, da @ db.T, rtol=0, atol=1e-12 * (np.abs(da) @ np.abs(db).T).max())
    assert np.allclose(absum, np.abs(da) @ np.abs(db).T, rtol=1e-12)
    ii, jj = np.array([0, 39, 5]), np.array([23, 0, 7])
    cs, _ = orc.mx_gemm(ac, as_, bc, bs, ii, jj)
    assert np.array_equal(cs, c[ii, jj])
