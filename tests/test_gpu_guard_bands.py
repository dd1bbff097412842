"""Guard bands: no kernel writes outside its outputs.

Every output is a view into the middle of a larger buffer whose margins (and,
where the call writes every element, the output itself) start as a sentinel
byte pattern.  After the call the margins must still hold the sentinel, and
outputs the call fully defines must hold none of it where a value was
expected.  Shapes are ragged: row counts that are not multiples of 128,
column counts that are not multiples of 256 or 512, GEMM extents that leave
partly covered tiles, and one 2-byte-aligned bf16 output."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quant_amd as nv
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
PAD = 4096  # bytes before and after each output
SENT = 0xFF  # all-ones: a NaN in fp32 and bf16, so finiteness shows an output was written


class Guarded:
    def __init__(self, shape, dtype, shift=0):
        esz = torch.empty(0, dtype=dtype).element_size()
        n = int(np.prod(shape))
        self.pad = (PAD + shift) // esz
        self.tail = PAD // esz
        self.n = n
        self.buf = torch.empty(self.pad + n + self.tail, dtype=dtype, device=DEV)
        self.buf.view(torch.uint8).fill_(SENT)
        self.t = self.buf[self.pad:self.pad + n].view(shape)

    def check(self, name):
        raw = self.buf.view(torch.uint8).cpu().numpy()
        esz = self.buf.element_size()
        head, tail = raw[:self.pad * esz], raw[(self.pad + self.n) * esz:]
        assert (head == SENT).all(), f"{name}: write before the output at byte {np.nonzero(head != SENT)[0][-1]}"
        assert (tail == SENT).all(), f"{name}: write after the output at byte {np.nonzero(tail != SENT)[0][0]}"


def quantized(rows, cols, transposed, block=16):
    q = dict(codes=Guarded((rows, cols // 2), torch.uint8), scales=Guarded((rows, cols // block), torch.uint8))
    if block == 16:
        q["tensor_scale"] = Guarded((2,), torch.float32)
    if transposed:
        q["codes_t"] = Guarded((cols, rows // 2), torch.uint8)
        q["scales_t"] = Guarded((cols, rows // 16), torch.uint8)
    return q


def check_all(q):
    for k, g in q.items():
        g.check(k)


def views(q):
    return {k: g.t for k, g in q.items()}


RAGGED = [(48, 80), (160, 272), (304, 400), (33, 2064), (144, 1040)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rounding,rht", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("shape", RAGGED)
def test_quantize_rowwise(shape, dtype, rounding, rht):
    x = datagen.sweep(*shape, seed=1).to(dtype).to(DEV)
    q = quantized(*shape, False)
    nv.nvfp4_quantize(x, rounding, 3, rht, 4, **views(q))
    torch.cuda.synchronize()
    check_all(q)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", [s for s in RAGGED if s[0] % 16 == 0])
def test_quantize_with_columnwise_copy_and_2d(shape, dtype, rounding):
    x = datagen.sweep(*shape, seed=2).to(dtype).to(DEV)
    q = quantized(*shape, True)
    nv.nvfp4_quantize(x, rounding, 3, 0, 0, **views(q))
    torch.cuda.synchronize()
    check_all(q)
    q2 = quantized(*shape, True)
    nv.nvfp4_quantize_2d(x, rounding, 3, **views(q2))
    torch.cuda.synchronize()
    check_all(q2)


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("rht_t", [0, 1])
@pytest.mark.parametrize("shape", [s for s in RAGGED if s[0] % 16 == 0])
def test_cast_transpose(shape, rounding, rht_t):
    x = datagen.grad(tokens=shape[0], out_features=shape[1], seed=3).to(DEV)
    q = quantized(*shape, False)
    qt = quantized(shape[1], shape[0], False)
    nv.nvfp4_quantize_cast_transpose(x, rounding, 5, 6, rht_t, 7, q["codes"].t, q["scales"].t,
                                     q["tensor_scale"].t, qt["codes"].t, qt["scales"].t, qt["tensor_scale"].t)
    torch.cuda.synchronize()
    check_all(q)
    check_all(qt)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_rht_and_dequantize(out_dtype):
    rows, cols = 33, 400
    x = datagen.sweep(rows, cols, seed=4).to(DEV)
    y = Guarded((rows, cols), torch.float32)
    nv.nvfp4_rht(x, 9, y.t)
    q = nv.quantize(x)
    out = Guarded((rows, cols), out_dtype)
    nv.nvfp4_dequantize(q.codes, q.scales, q.tensor_scale, rows, cols, out.t)
    torch.cuda.synchronize()
    y.check("rht y")
    out.check("dequantize out")
    assert torch.isfinite(y.t).all() and torch.isfinite(out.t.float()).all()


@pytest.mark.parametrize("M,N,K", [(200, 136, 272), (130, 250, 512), (256, 512, 512), (8448, 2816, 512),
                                   (17, 300, 48)])
def test_gemm_and_gemm_ex(M, N, K):
    a = nv.quantize(datagen.act(tokens=M, hidden=K, seed=5).to(DEV))
    b = nv.quantize(datagen.weight(out_features=N, in_features=K, seed=6).to(DEV), rounding=1, seed=2)
    c = Guarded((M, N), torch.float32)
    nv.gemm(a, b, out=c.t)
    torch.cuda.synchronize()
    c.check("gemm C")
    assert torch.isfinite(c.t).all()  # every output written (the sentinel is a NaN)
    for dtype, shift in ((torch.bfloat16, 0), (torch.bfloat16, 2), (torch.float32, 0)):
        for beta in (0.0, 0.5):
            ce = Guarded((M, N), dtype, shift)
            if beta:
                ce.t.fill_(1.0)
            amax = Guarded((1,), torch.float32)
            nv.gemm_ex(a, b, out=ce.t, beta=beta, amax=amax.t)
            torch.cuda.synchronize()
            ce.check(f"gemm_ex C {dtype} shift {shift} beta {beta}")
            amax.check("gemm_ex amax")
            assert torch.isfinite(ce.t.float()).all()


@pytest.mark.parametrize("M,N,K", [(96, 160, 96), (256, 256, 256), (300, 260, 128)])
def test_mxfp4(M, N, K):
    a = datagen.act(tokens=M, hidden=K, seed=7).to(DEV)
    b = datagen.weight(out_features=N, in_features=K, seed=8).to(DEV)
    qa, qb = quantized(M, K, False, block=32), quantized(N, K, False, block=32)
    nv.mxfp4_quantize(a, qa["codes"].t, qa["scales"].t)
    nv.mxfp4_quantize(b, qb["codes"].t, qb["scales"].t)
    torch.cuda.synchronize()
    check_all(qa)
    check_all(qb)
    c = Guarded((M, N), torch.float32)
    nv.mxfp4_gemm(qa["codes"].t, qa["scales"].t, qb["codes"].t, qb["scales"].t, M, N, K, c.t)
    out = Guarded((M, K), torch.bfloat16)
    nv.mxfp4_dequantize(qa["codes"].t, qa["scales"].t, M, K, out.t)
    torch.cuda.synchronize()
    c.check("mxfp4 C")
    out.check("mxfp4 dequantize")
    assert torch.isfinite(c.t).all()
