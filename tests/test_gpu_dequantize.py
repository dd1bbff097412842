"""GPU parity of nvfp4_dequantize against the oracle's dequantization.

The oracle computes e2m1(code) * e4m3(scale) / S_enc in double; the product
is exact and the quotient of two fp32 values rounded to double and then to
fp32 is the correctly rounded fp32 quotient, so the fp32 output must match
float32(oracle) bit for bit (signed zeros included), and the bf16 output
must match that fp32 value rounded to nearest-even bf16 (torch's CPU cast).
Inputs are codes written here or by the oracle's quantizers, never by the
GPU path."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quant_amd as nv
import oracle
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def run(codes, scales, s_enc, dtype):
    rows, cols = codes.shape[0], codes.shape[1] * 2
    q = nv.Quantized(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.tensor([s_enc, 0.0], dtype=torch.float32, device=DEV))
    out = nv.dequantize(q, dtype=dtype)
    torch.cuda.synchronize()
    return out.cpu()


def expect(codes, scales, s_enc, dtype):
    # a tiny tensor scale takes some values past fp32's range: the cast rounds
    # them to infinity, as the kernel's single division does (the overflow is
    # the expected result, not a warning)
    with np.errstate(over="ignore"):
        ref32 = torch.from_numpy(oracle.dequantize(codes, scales, s_enc).astype(np.float32))
    return ref32 if dtype == torch.float32 else ref32.to(torch.bfloat16)


def same_bits(a, b):
    ia = a.view(torch.int32 if a.dtype == torch.float32 else torch.int16)
    ib = b.view(torch.int32 if b.dtype == torch.float32 else torch.int16)
    bad = torch.nonzero(ia != ib)
    assert bad.numel() == 0, f"{bad.shape[0]} mismatches, first at {bad[:4].tolist()}: " \
                             f"{a[tuple(bad[0])]} vs {b[tuple(bad[0])]}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("s_enc", [1.0, 2688.0 / 3.7, 3.4028234663852886e38, 7.899e-36, 0.3])
def test_every_code_and_scale_byte(s_enc, dtype):
    # row b: scale byte b (0x00 .. 0x7E) on both blocks, codes 0..15 twice
    nb = 0x7F
    row = np.array([c | (c + 1) << 4 for c in range(0, 16, 2)] * 2, dtype=np.uint8)  # 16 codes x 2
    codes = np.tile(row, (nb, 1))
    scales = np.repeat(np.arange(nb, dtype=np.uint8)[:, None], 2, axis=1)
    s_enc = float(np.float32(s_enc))
    same_bits(run(codes, scales, s_enc, dtype), expect(codes, scales, s_enc, dtype))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_quantized_tensors(dtype):
    cases = []
    g = datagen.host_input(datagen.grad(tokens=304, out_features=400, seed=2))
    cases.append(oracle.quantize_1d(g, rounding=1, seed=3)[:3])
    w = datagen.host_input(datagen.weight(out_features=160, in_features=272, seed=1))
    q2 = oracle.quantize_2d(w)
    cases += [q2[:3], (q2[3], q2[4], q2[2])]
    x = datagen.host_input(datagen.act(tokens=48, hidden=80, seed=5))
    qt = oracle.quantize_1d(np.ascontiguousarray(x.T), rht=1, rht_seed=9)
    cases.append(qt[:3])
    cases.append(oracle.quantize_1d(np.ones((1, 16), np.float32))[:3])
    for codes, scales, ts in cases:
        same_bits(run(codes, scales, float(ts[0]), dtype), expect(codes, scales, float(ts[0]), dtype))


@pytest.mark.timeout(600)
def test_dequantize_full_size_activation():
    x = datagen.host_input(datagen.act())
    codes, scales, ts, _, _ = oracle.quantize_1d(x)
    for dtype in (torch.float32, torch.bfloat16):
        same_bits(run(codes, scales, float(ts[0]), dtype), expect(codes, scales, float(ts[0]), dtype))
