"""GPU parity of the cast-transpose: one read of x per pass, two NVFP4 copies.

The rowwise copy must equal the oracle's 1D quantization of x, and the
columnwise copy the oracle's 1D quantization of x^T under its own seed (with
the Hadamard transform of "Pretraining Large Language Models with NVFP4",
2B.2, when rht_t), bit for bit: codes, scale bytes and both tensor-scale
floats of each copy.  Small cases span several 128 x 512 tiles with ragged
row and column tails; the full-size cases are the activation X [8192 x 5120]
(RNE, transform on X^T) and the gradient dY [8192 x 20480] (SR, transform on
dY^T) of the linear layer, compared over the whole tensor."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quant_amd as nv
import oracle
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def host(t):
    return t.detach().cpu().numpy()


def assert_same(q, ref, what):
    assert np.array_equal(host(q.tensor_scale), ref[2]), (what, host(q.tensor_scale), ref[2])
    for name, got, want in (("codes", q.codes, ref[0]), ("scales", q.scales, ref[1])):
        bad = np.argwhere(host(got) != want)
        assert bad.size == 0, f"{what} {name}: {len(bad)} mismatches, first at {bad[:4].tolist()}"


def oracle_pair(xh, rounding, seed, seed_t, rht_t, rht_seed):
    row = oracle.quantize_1d(xh, rounding=rounding, seed=seed)
    col = oracle.quantize_1d(np.ascontiguousarray(xh.T), rounding=rounding, seed=seed_t, rht=rht_t,
                             rht_seed=rht_seed)
    return row, col


SMALL = [(16, 16), (48, 80), (128, 512), (160, 272), (304, 1040), (144, 528), (256, 4096),
         (1024, 1536), (4096, 16), (16, 8192)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("rht_t", [0, 1])
@pytest.mark.parametrize("shape", SMALL)
def test_cast_transpose_small(shape, rht_t, rounding, dtype):
    x = datagen.grad(tokens=shape[0], out_features=shape[1], seed=shape[1])
    x = x.float() if dtype == "f32" else x
    q, qt = nv.quantize_cast_transpose(x.to(DEV), rounding=rounding, seed=5, seed_t=6, rht_t=bool(rht_t),
                                       rht_seed=77)
    torch.cuda.synchronize()
    row, col = oracle_pair(datagen.host_input(x), rounding, 5, 6, rht_t, 77)
    assert_same(q, row, "rowwise")
    assert_same(qt, col, "columnwise")


def test_cast_transpose_edge_values_and_reuse():
    # a zero tensor, blocks of -0, a lone outlier, subnormal magnitudes
    x = torch.zeros(64, 96)
    x[16:32, :48] = -0.0
    x[40, 70] = 3000.0
    x[48:64, 16:32] = 1e-40
    for rounding in (0, 1):
        for rht_t in (0, 1):
            for t in (torch.zeros(32, 64), x):
                q, qt = nv.quantize_cast_transpose(t.to(DEV), rounding=rounding, seed=2, seed_t=3,
                                                   rht_t=bool(rht_t), rht_seed=9)
                torch.cuda.synchronize()
                row, col = oracle_pair(t.numpy(), rounding, 2, 3, rht_t, 9)
                assert_same(q, row, "rowwise")
                assert_same(qt, col, "columnwise")
    # the same output buffers reused: the amax targets are cleared by each call
    y = datagen.grad(tokens=256, out_features=512, seed=1).to(DEV)
    q, qt = nv.quantize_cast_transpose(y, rounding=1, seed=4, seed_t=5)
    nv.nvfp4_quantize_cast_transpose(y * 0.01, 1, 4, 5, 1, 0, q.codes, q.scales, q.tensor_scale, qt.codes,
                                     qt.scales, qt.tensor_scale)
    torch.cuda.synchronize()
    row, col = oracle_pair(datagen.host_input((y * 0.01).cpu()), 1, 4, 5, 1, 0)
    assert_same(q, row, "rowwise")
    assert_same(qt, col, "columnwise")


def test_cast_transpose_equals_composed_calls():
    x = datagen.grad(tokens=512, out_features=2048, seed=3).to(DEV)
    q, qt = nv.quantize_cast_transpose(x, rounding=1, seed=10, seed_t=11, rht_t=True, rht_seed=12)
    a = nv.quantize(x, rounding=1, seed=10)
    b = nv.quantize(x.t().contiguous(), rounding=1, seed=11, rht=True, rht_seed=12)
    torch.cuda.synchronize()
    for u, v in ((q.codes, a.codes), (q.scales, a.scales), (q.tensor_scale, a.tensor_scale),
                 (qt.codes, b.codes), (qt.scales, b.scales), (qt.tensor_scale, b.tensor_scale)):
        assert torch.equal(u, v)


FULL = [
    ("X_rne_rht", lambda: datagen.act(DEV), 0),
    ("dY_sr_rht", lambda: datagen.grad(DEV), 1),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,gen,rounding", FULL, ids=[f[0] for f in FULL])
def test_cast_transpose_full_size(name, gen, rounding):
    x = gen()
    q, qt = nv.quantize_cast_transpose(x, rounding=rounding, seed=0, seed_t=0, rht_t=True, rht_seed=0)
    torch.cuda.synchronize()
    row, col = oracle_pair(datagen.host_input(x), rounding, 0, 0, 1, 0)
    assert_same(q, row, "rowwise")
    assert_same(qt, col, "columnwise")


@pytest.mark.timeout(900)
def test_cast_transpose_more_than_2_31_elements():
    """A 16400 x 131072 gradient-like bf16 tensor (2^31 + 2^24 elements) through
    the cast-transpose with SR and the transform on the columnwise copy, both
    copies bit for bit against the oracle: offsets and SR draw indices pass
    2^31 in both layouts."""
    x = datagen.grad(DEV, seed=4, tokens=16400, out_features=131072)
    assert x.numel() > 2 ** 31
    q, qt = nv.quantize_cast_transpose(x, rounding=1, seed=5, seed_t=6, rht_t=True, rht_seed=77)
    torch.cuda.synchronize()
    xh = datagen.host_input(x)
    del x
    row, col = oracle_pair(xh, 1, 5, 6, 1, 77)
    assert_same(q, row, "rowwise")
    assert_same(qt, col, "columnwise")
