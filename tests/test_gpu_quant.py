"""GPU parity of the quantizer and the Hadamard transform against the oracle.

Codes, scale bytes and both tensor-scale floats must be bit-identical.  Small
cases span several 128x128 tiles with ragged tails; the full-size cases are
the workload's tensors (fprop X and W, dgrad dY, wgrad dY^T and X^T, and the
quantizer sweep), compared over the whole tensor."""
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


def assert_same(q, ref, transposed):
    assert np.array_equal(host(q.tensor_scale), ref[2]), (host(q.tensor_scale), ref[2])
    for name, got, want in (("codes", q.codes, ref[0]), ("scales", q.scales, ref[1])):
        g = host(got)
        bad = np.argwhere(g != want)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:4].tolist()}"
    if transposed:
        for name, got, want in (("codes_t", q.codes_t, ref[3]), ("scales_t", q.scales_t, ref[4])):
            g = host(got)
            bad = np.argwhere(g != want)
            assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:4].tolist()}"


def make(rows, cols, dtype, seed=0, kind="sweep"):
    if kind == "sweep":
        t = datagen.sweep(rows, cols, seed=seed)
    elif kind == "grad":
        t = datagen.grad(tokens=rows, out_features=cols, seed=seed)
    else:
        t = datagen.act(tokens=rows, hidden=cols, seed=seed)
    return t.float() if dtype == "f32" else t


SMALL = [(16, 16), (48, 80), (128, 128), (160, 272), (304, 400), (256, 4096)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", SMALL + [(300, 400), (7, 48), (1, 16), (33, 2064)])
def test_quantize_rowwise(shape, dtype, rounding):
    x = make(*shape, dtype, seed=shape[0])
    q = nv.quantize(x.to(DEV), rounding=rounding, seed=11)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(datagen.host_input(x), rounding=rounding, seed=11)
    assert_same(q, ref, False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", SMALL + [(400, 1040), (272, 1552), (4096, 16), (16, 8192)])
def test_quantize_columnwise(shape, dtype, rounding):
    x = make(*shape, dtype, seed=shape[1], kind="act")
    q = nv.quantize(x.to(DEV), rounding=rounding, seed=5, transposed=True)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(datagen.host_input(x), rounding=rounding, seed=5, transposed=True)
    assert_same(q, ref, True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", SMALL + [(400, 48), (384, 512), (4096, 16), (16, 8192)])
def test_quantize_2d(shape, dtype, rounding):
    w = datagen.weight(out_features=shape[0], in_features=shape[1], seed=shape[0] + shape[1])
    w = w.float() if dtype == "f32" else w
    q = nv.quantize_2d(w.to(DEV), rounding=rounding, seed=9)
    torch.cuda.synchronize()
    ref = oracle.quantize_2d(datagen.host_input(w), rounding=rounding, seed=9)
    assert_same(q, ref, True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (300, 400), (64, 8192)])
def test_quantize_rht(shape, dtype, rounding):
    x = make(*shape, dtype, seed=3, kind="grad")
    q = nv.quantize(x.to(DEV), rounding=rounding, seed=2, rht=True, rht_seed=77)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(datagen.host_input(x), rounding=rounding, seed=2, rht=1, rht_seed=77)
    assert_same(q, ref, False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rht_standalone_and_fused_equals_composed(dtype):
    x = make(96, 320, dtype, seed=4, kind="grad").to(DEV)
    y = nv.rht(x, rht_seed=123)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), oracle.rht(datagen.host_input(x.cpu()), 123))
    fused = nv.quantize(x, rounding=1, seed=8, rht=True, rht_seed=123)
    comp = nv.quantize(y, rounding=1, seed=8)
    torch.cuda.synchronize()
    for a, b in ((fused.codes, comp.codes), (fused.scales, comp.scales),
                 (fused.tensor_scale, comp.tensor_scale)):
        assert torch.equal(a, b)


def test_edge_cases():
    cases = {
        "zeros": torch.zeros(32, 64),
        "neg_zero_blocks": torch.cat([torch.full((16, 32), -0.0), torch.ones(16, 32)], 0),
        "tiny_amax": torch.full((16, 32), 1e-40),
        "huge": torch.full((16, 32), 3e38),
        "ties": torch.tensor([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4).reshape(1, 32)
                .repeat(16, 1).contiguous(),
        "one_outlier": torch.cat([torch.full((16, 16), 1e-3), torch.full((16, 16), 2688.0)], 1),
        # S_enc and a block multiplier overflow binary32 and clamp to FLT_MAX
        "clamped_multiplier": torch.zeros(16, 32).index_put_(
            (torch.tensor([0, 0, 0, 0, 5]), torch.tensor([0, 16, 17, 18, 20])),
            torch.tensor([2.0 ** -120, 2.0 ** -128, 2.0 ** -130, -(2.0 ** -129), 2.0 ** -127])),
        # blocks whose E4M3 scale rounds to zero, holding values up to 3
        "zero_scale_blocks": torch.cat([torch.full((16, 16), 2.0 ** 40),
                                        torch.linspace(-3.0, 3.0, 256).reshape(16, 16)], 1),
    }
    for name, x in cases.items():
        x = x.float().contiguous()
        for rounding in (0, 1):
            q = nv.quantize(x.to(DEV), rounding=rounding, seed=1, transposed=True)
            q2 = nv.quantize_2d(x.to(DEV), rounding=rounding, seed=1)
            torch.cuda.synchronize()
            assert_same(q, oracle.quantize_1d(x.numpy(), rounding=rounding, seed=1, transposed=True),
                        True)
            assert_same(q2, oracle.quantize_2d(x.numpy(), rounding=rounding, seed=1), True)


def test_deterministic_and_reusable_outputs():
    x = make(256, 512, "bf16", seed=9).to(DEV)
    a = nv.quantize(x, rounding=1, seed=4, transposed=True)
    b = nv.quantize(x, rounding=1, seed=4, transposed=True)
    torch.cuda.synchronize()
    for u, v in ((a.codes, b.codes), (a.codes_t, b.codes_t), (a.scales, b.scales)):
        assert torch.equal(u, v)
    # the same output buffers reused for a tensor with a smaller amax
    nv.nvfp4_quantize(x * 0.001, 0, 0, 0, 0, a.codes, a.scales, a.tensor_scale)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(datagen.host_input((x * 0.001).cpu()))
    assert np.array_equal(host(a.codes), ref[0]) and np.array_equal(host(a.tensor_scale), ref[2])


# ---------------------------------------------------------------- full size
FULL = [
    ("fprop_X_1d_rne", lambda: datagen.act(DEV), dict(rounding=0)),
    ("dgrad_dY_1d_sr", lambda: datagen.grad(DEV), dict(rounding=1, seed=0)),
    ("wgrad_dYt_1d_sr_rht", lambda: datagen.grad(DEV).t().contiguous(),
     dict(rounding=1, seed=0, rht=1, rht_seed=0)),
    ("wgrad_Xt_1d_rne_rht", lambda: datagen.act(DEV).t().contiguous(),
     dict(rounding=0, rht=1, rht_seed=0)),
]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,gen,kw", FULL, ids=[f[0] for f in FULL])
def test_full_size_1d(name, gen, kw):
    x = gen()
    q = nv.quantize(x, rounding=kw.get("rounding", 0), seed=kw.get("seed", 0),
                    rht=bool(kw.get("rht", 0)), rht_seed=kw.get("rht_seed", 0))
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(datagen.host_input(x), **kw)
    assert_same(q, ref, False)


@pytest.mark.timeout(900)
def test_full_size_weight_2d_and_transpose_identity():
    w = datagen.weight(DEV)
    q = nv.quantize_2d(w)
    torch.cuda.synchronize()
    ref = oracle.quantize_2d(datagen.host_input(w))
    assert_same(q, ref, True)
    # W^T quantized on its own gives the transposed copy, bit for bit
    qt = nv.quantize_2d(w.t().contiguous(), transposed=False)
    torch.cuda.synchronize()
    assert torch.equal(qt.codes, q.codes_t) and torch.equal(qt.scales, q.scales_t)


SWEEP = [(r, c, two_d, rnd) for (r, c) in ((8192, 5120), (8192, 20480), (32768, 5120))
         for two_d in (False, True) for rnd in (0, 1)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("rows,cols,two_d,rounding", SWEEP)
def test_full_size_sweep(rows, cols, two_d, rounding):
    x = datagen.sweep(rows, cols, device=DEV)
    if two_d:
        q = nv.quantize_2d(x, rounding=rounding, seed=0)
        torch.cuda.synchronize()
        ref = oracle.quantize_2d(datagen.host_input(x), rounding=rounding, seed=0)
    else:
        q = nv.quantize(x, rounding=rounding, seed=0, transposed=True)
        torch.cuda.synchronize()
        ref = oracle.quantize_1d(datagen.host_input(x), rounding=rounding, seed=0, transposed=True)
    assert_same(q, ref, True)


@pytest.mark.timeout(900)
def test_more_than_2_31_elements():
    """A 16400 x 131072 bf16 tensor (2^31 + 2^24 elements, 4.3 GB) quantized
    1D with SR and its columnwise copy, bit for bit against the oracle: every
    element offset, code byte offset and SR draw index passes 2^31."""
    x = datagen.act(DEV, seed=5, tokens=16400, hidden=131072)
    assert x.numel() > 2 ** 31
    q = nv.quantize(x, rounding=1, seed=3, transposed=True)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(datagen.host_input(x), rounding=1, seed=3, transposed=True)
    assert_same(q, ref, True)
