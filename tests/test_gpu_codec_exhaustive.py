"""Exhaustive check of the device element encoder through the public C ABI.

Every block is [6.0, x1 .. x15] and one extra row holds 2688, so S_enc = 1,
every block scale byte is 0x38 (1.0), the multiplier is exactly 1 and the
kernel encodes y = x.  The x run over every fp32 bit pattern with
2^-9 <= |x| <= 6 (both signs; every tie, grid point and SR threshold of the
E2M1 grid lies there) plus a random sample of smaller magnitudes down to
subnormals, and the codes must equal the oracle's codec (argmin with the
tie rule, or the SR rule with the oracle's Philox draws) bit for bit."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quant_amd as nv
import oracle

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
CHUNK = 15 * (1 << 20)  # values per launch


def patterns():
    lo, hi = np.uint32(118 << 23), np.uint32(0x40C00000)  # 2^-9 .. 6.0 inclusive
    core = np.arange(lo, hi + np.uint32(1), dtype=np.uint32)
    rng = np.random.default_rng(0)
    small = rng.integers(0, 118 << 23, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    pos = np.concatenate([core, small, np.array([0], np.uint32)])
    return pos


def run_chunk(vals, rounding, seed):
    n = vals.size
    rows = -(-n // 15)
    x = np.zeros((rows + 1, 16), dtype=np.float32)
    x[:rows, 0] = 6.0
    body = np.zeros(rows * 15, dtype=np.float32)
    body[:n] = vals
    x[:rows, 1:] = body.reshape(rows, 15)
    x[rows, 0] = 2688.0
    q = nv.quantize(torch.from_numpy(x).to(DEV), rounding=rounding, seed=seed)
    torch.cuda.synchronize()
    ts = q.tensor_scale.cpu().numpy()
    assert ts[0] == 1.0 and ts[1] == 2688.0
    scales = q.scales.cpu().numpy()
    assert (scales[:rows] == 0x38).all()
    c = q.codes.cpu().numpy()
    codes = np.stack([c & 15, c >> 4], -1).reshape(rows + 1, 16)
    assert (codes[:rows, 0] == 7).all()
    got = codes[:rows, 1:].reshape(-1)[:n]
    y = x[:rows, 1:].reshape(-1)[:n]
    if rounding == 0:
        want = oracle.e2m1_encode_rne_n(y)
    else:
        u = oracle.sr_bits_n(seed, 0, 0, (rows + 1) * 16).reshape(rows + 1, 16)[:rows, 1:]
        want = oracle.e2m1_encode_sr_n(y, u.reshape(-1)[:n])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{bad.size} mismatches, e.g. y={y[bad[:4]]} got={got[bad[:4]]} "
                           f"want={want[bad[:4]]}")


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("rounding", [0, 1])
def test_device_encoder_exhaustive(rounding):
    pos = patterns()
    for sign in (np.uint32(0), np.uint32(0x80000000)):
        allv = (pos | sign).view(np.float32)
        for k in range(0, allv.size, CHUNK):
            run_chunk(allv[k:k + CHUNK], rounding, seed=17 + k)


# E2M1 grid intervals [lo, hi) between neighbouring magnitudes
INTERVALS = [(0.0, 0.5), (0.5, 1.0), (1.0, 1.5), (1.5, 2.0), (2.0, 3.0), (3.0, 4.0), (4.0, 6.0)]


def encode_layout(body, first=6.0):
    """rows of [first, 15 test values] plus a last row whose 2688 sets
    S_enc = 1: every block's scale byte is then 0x38 (1.0) and y = x."""
    n = body.size
    rows = -(-n // 15)
    x = np.zeros((rows + 1, 16), dtype=np.float32)
    x[:rows, 0] = first
    flat = np.zeros(rows * 15, dtype=np.float32)
    flat[:n] = body
    x[:rows, 1:] = flat.reshape(rows, 15)
    x[rows, 0] = 2688.0
    return x, rows


def device_codes(x, rows, rounding, seed):
    q = nv.quantize(torch.from_numpy(x).to(DEV), rounding=rounding, seed=seed)
    torch.cuda.synchronize()
    assert np.array_equal(q.tensor_scale.cpu().numpy(), np.array([1.0, 2688.0], np.float32))
    assert (q.scales.cpu().numpy()[:rows] == 0x38).all()
    c = q.codes.cpu().numpy()
    return np.stack([c & 15, c >> 4], -1).reshape(rows + 1, 16)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_device_sr_exact_thresholds(sign):
    """Stochastic rounding at its exact thresholds, for the draw each element
    actually gets.  Element i (row-major index of the tensor) draws
    u_i = the oracle's 16-bit Philox value for (seed, stream 0, i).  Its value
    is planted at y = lo + (hi - lo) * u_i / 2^16, exactly on the threshold,
    where "u < f * 2^16" is false (round down to lo), or at the next float
    above it, where it is true (round up to hi): the SR example of the pages
    (a value between two grid points goes up with probability equal to its
    fractional distance) at the one point where a comparison off by one ulp
    or one bit would show."""
    seed = 23
    n_rows = 1 << 16
    idx = np.arange(n_rows * 16, dtype=np.int64).reshape(n_rows, 16)[:, 1:].reshape(-1)
    u = oracle.sr_bits_n(seed, 0, 0, (n_rows + 1) * 16).astype(np.int64)[idx]
    k = np.arange(idx.size)
    lo = np.array([iv[0] for iv in INTERVALS])[k % 7]
    hi = np.array([iv[1] for iv in INTERVALS])[k % 7]
    y = (lo + (hi - lo) * u / 65536.0).astype(np.float32)
    assert np.array_equal(y.astype(np.float64), lo + (hi - lo) * u / 65536.0)  # planted exactly
    up = (k // 7) % 2 == 1
    y = np.where(up, np.nextafter(y, np.float32(np.inf)), y).astype(np.float32)
    x, rows = encode_layout(sign * y)
    assert rows == n_rows
    got = device_codes(x, rows, 1, seed)[:rows, 1:].reshape(-1)
    want = oracle.e2m1_encode_sr_n(sign * y, u.astype(np.uint16))
    # the oracle's own rule lands on lo at the threshold and on hi just above it
    mag = np.array([oracle.e2m1_value(int(c)) for c in range(8)])[want & 7]
    assert np.array_equal(mag, np.where(up, hi, lo))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f"{bad.size} mismatches, e.g. y={y[bad[:4]]} u={u[bad[:4]]} got={got[bad[:4]]} "
                           f"want={want[bad[:4]]}")


@pytest.mark.parametrize("rounding", [0, 1])
def test_device_encoder_saturation_range(rounding):
    """Every fp32 magnitude in (6, 6.375] of both signs, where E2M1 saturates
    at 6 (values of this size occur whenever a block's E4M3 scale rounds
    down).  The block maximum 6.375 gives s = 6.375 / 6 = 1.0625, a tie
    between the E4M3 values 1 and 1.125 that goes to the even 1, so y = x."""
    lo, hi = np.uint32(0x40C00001), np.uint32(0x40CC0000)  # next after 6.0 .. 6.375
    mags = np.arange(lo, hi + np.uint32(1), dtype=np.uint32).view(np.float32)
    body = np.concatenate([mags, -mags])
    x, rows = encode_layout(body, first=6.375)
    got = device_codes(x, rows, rounding, 31)[:rows, 1:].reshape(-1)[:body.size]
    if rounding == 0:
        want = oracle.e2m1_encode_rne_n(body)
    else:
        u = oracle.sr_bits_n(31, 0, 0, (rows + 1) * 16).reshape(rows + 1, 16)[:rows, 1:].reshape(-1)
        want = oracle.e2m1_encode_sr_n(body, u[:body.size])
    assert np.array_equal(want & 7, np.full(body.size, 7))  # saturated: magnitude 6
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, e.g. y={body[bad[:4]]} got={got[bad[:4]]}"


@pytest.mark.timeout(600)
def test_block_scale_bytes_at_every_e4m3_boundary():
    """The block scale byte (E4M3 of amax_b * S_enc / 6, round to nearest
    even, saturating at 448) around every rounding boundary of E4M3: rows
    [a, 0, ..., 0] with a tensor maximum of 2688 elsewhere (S_enc = 1), so the
    byte is E4M3(fl(a / 6)).  For every midpoint m between neighbouring E4M3
    values (and the saturation point 464), a runs over the 257 fp32 values
    around fl(6 m); plus a million random block maxima in (0, 2688].  Scale
    bytes and codes must equal the oracle's."""
    vals = np.array(sorted({oracle.e4m3_value(b) for b in range(0x7F)}))
    mids = np.concatenate([(vals[:-1] + vals[1:]) / 2, [464.0]])
    centers = (6.0 * mids).astype(np.float32).view(np.int32)
    near = (centers[:, None] + np.arange(-128, 129)[None, :]).reshape(-1)
    near = near[(near > 0) & (near <= np.float32(2688.0).view(np.int32))].view(np.float32)
    rng = np.random.default_rng(5)
    rand = rng.uniform(0.0, 2688.0, 1 << 20).astype(np.float32)
    rand = np.concatenate([rand, np.exp2(rng.uniform(-40, 11.39, 1 << 18)).astype(np.float32)])
    a = np.concatenate([near, rand])
    a = a[(a > 0) & (a <= 2688.0)]
    x = np.zeros((a.size + 1, 16), dtype=np.float32)
    x[:-1, 0] = a
    x[-1, 0] = 2688.0
    q = nv.quantize(torch.from_numpy(x).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(x)
    assert ref[2][0] == 1.0
    for got, want, name in ((q.scales, ref[1], "scales"), (q.codes, ref[0], "codes")):
        g = got.cpu().numpy()
        bad = np.argwhere(g != want)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, e.g. a={a[bad[:4, 0]]} got={g[tuple(bad[:4].T)]}"
