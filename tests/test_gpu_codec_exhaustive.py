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
