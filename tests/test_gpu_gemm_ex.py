"""GPU checks of the GEMM epilogue options (nvfp4_gemm_ex: bf16 output,
beta-accumulation, output amax) and of the single-read quantizer
(nvfp4_quantize_with_amax).

GEMM results are compared with the oracle's double-precision product of the
oracle's quantizations ("NVIDIA acelera el preentrenamiento de LLM",
"Como Funciona Mixed-Precision con NVFP4": BF16 or FP32 accumulators and
outputs): within 1e-5 * sum|ab| plus the output's own rounding (2^-8 of the
value for bf16, 2^-22 for the fp32 add of beta * C_old).  The amax must
equal the maximum |C| of the stored output exactly.  The single-read
quantizer, given the amax computed on the host, must equal the oracle's
quantization bit for bit."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quant_amd as nv
import oracle
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def operands(M, N, K, seed):
    a = datagen.host_input(datagen.act(tokens=M, hidden=K, seed=seed))
    b = datagen.host_input(datagen.weight(out_features=N, in_features=K, seed=seed + 1))
    qa, qb = oracle.quantize_1d(a), oracle.quantize_1d(b)
    up = lambda q: nv.Quantized(torch.from_numpy(q[0]).to(DEV), torch.from_numpy(q[1]).to(DEV),
                                torch.from_numpy(q[2]).to(DEV))
    ref, absum = oracle.gemm(qa[0], qa[1], qa[2][0], qb[0], qb[1], qb[2][0])
    return up(qa), up(qb), ref, absum


SHAPES = [(256, 256, 512), (512, 256, 1024), (100, 70, 96), (256, 512, 448)]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_gemm_ex(M, N, K, dtype, beta):
    a, b, ref, absum = operands(M, N, K, seed=M + K)
    g = torch.Generator().manual_seed(3)
    c_in = (torch.randn(M, N, generator=g) * float(np.abs(ref).max())).to(dtype)
    c = c_in.to(DEV)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)  # overwritten by the call
    nv.gemm_ex(a, b, out=c, beta=beta, amax=amax)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy().astype(np.float64)
    want = ref + beta * c_in.float().numpy().astype(np.float64)
    bound = 1e-5 * absum + 2.0 ** -22 * (np.abs(ref) + np.abs(beta * c_in.float().numpy()))
    if dtype == torch.bfloat16:  # rounding the fp32 value to bf16: at most 2^-9 of it
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(want)
    excess = np.abs(got - want) - bound
    assert excess.max() <= 0, f"max excess {excess.max()} at {np.unravel_index(excess.argmax(), excess.shape)}"
    assert amax.item() == float(np.abs(c.float().cpu().numpy()).max())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_gemm_ex_whole_waves(dtype, beta):
    # 256 tiles of 256 x 256: the whole-wave kernel (the shapes above run as
    # 256 x 128 halves); sampled outputs against the oracle, the amax exactly
    M, N, K = 4096, 4096, 512
    ah = datagen.host_input(datagen.act(tokens=M, hidden=K, seed=21))
    bh = datagen.host_input(datagen.weight(out_features=N, in_features=K, seed=22))
    qa, qb = oracle.quantize_1d(ah), oracle.quantize_1d(bh)
    up = lambda q: nv.Quantized(torch.from_numpy(q[0]).to(DEV), torch.from_numpy(q[1]).to(DEV),
                                torch.from_numpy(q[2]).to(DEV))
    rng = np.random.default_rng(5)
    ii = np.concatenate([[0, M - 1, 0, M - 1], rng.integers(0, M, 3000)]).astype(np.int64)
    jj = np.concatenate([[0, 0, N - 1, N - 1], rng.integers(0, N, 3000)]).astype(np.int64)
    ref, absum = oracle.gemm_sample(qa[0], qa[1], qa[2][0], qb[0], qb[1], qb[2][0], ii, jj)
    g = torch.Generator().manual_seed(4)
    c_in = (torch.randn(M, N, generator=g) * float(np.abs(ref).max())).to(dtype)
    c = c_in.to(DEV)
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    nv.gemm_ex(up(qa), up(qb), out=c, beta=beta, amax=amax)
    torch.cuda.synchronize()
    got = c.float().cpu().numpy()[ii, jj].astype(np.float64)
    cin = c_in.float().numpy()[ii, jj].astype(np.float64)
    want = ref + beta * cin
    bound = 1e-5 * absum + 2.0 ** -22 * (np.abs(ref) + np.abs(beta * cin))
    if dtype == torch.bfloat16:
        bound = bound * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(want)
    excess = np.abs(got - want) - bound
    assert excess.max() <= 0, f"max excess {excess.max()} at sample {excess.argmax()}"
    assert amax.item() == float(c.float().abs().max().item())


@pytest.mark.parametrize("rounding,rht", [(0, 0), (1, 0), (1, 1)])
def test_quantize_with_amax_equals_oracle(rounding, rht):
    x = datagen.grad(tokens=304, out_features=1024, seed=7)
    xh = datagen.host_input(x)
    amax = np.abs(oracle.rht(xh, 5)).max() if rht else np.abs(x.float().numpy()).max()
    codes = torch.empty(304, 512, dtype=torch.uint8, device=DEV)
    scales = torch.empty(304, 64, dtype=torch.uint8, device=DEV)
    ts = torch.tensor([0.0, float(amax)], dtype=torch.float32, device=DEV)
    nv.nvfp4_quantize_with_amax(x.to(DEV), rounding, 9, rht, 5, codes, scales, ts)
    torch.cuda.synchronize()
    ref = oracle.quantize_1d(xh, rounding=rounding, seed=9, rht=rht, rht_seed=5)
    assert np.array_equal(ts.cpu().numpy(), ref[2])
    assert np.array_equal(codes.cpu().numpy(), ref[0]) and np.array_equal(scales.cpu().numpy(), ref[1])


def test_gemm_amax_feeds_single_read_quantizer():
    # the GEMM's bf16 output and amax, quantized in one read, equal the
    # two-pass quantization of the same output
    a, b, _, _ = operands(512, 1024, 512, seed=11)
    ts = torch.zeros(2, dtype=torch.float32, device=DEV)
    c = nv.gemm_ex(a, b, dtype=torch.bfloat16, amax=ts[1:])
    q1 = nv.Quantized(torch.empty(512, 512, dtype=torch.uint8, device=DEV),
                      torch.empty(512, 64, dtype=torch.uint8, device=DEV), ts)
    nv.nvfp4_quantize_with_amax(c, 1, 3, 0, 0, q1.codes, q1.scales, q1.tensor_scale)
    q2 = nv.quantize(c, rounding=1, seed=3)
    torch.cuda.synchronize()
    for u, v in ((q1.codes, q2.codes), (q1.scales, q2.scales), (q1.tensor_scale, q2.tensor_scale)):
        assert torch.equal(u, v)


@pytest.mark.parametrize("M,N,K,sampled", [(512, 256, 1024, False), (4096, 4096, 512, True)])
@pytest.mark.parametrize("beta", [0.0, 0.5])
def test_gemm_ex_bf16_output_two_byte_aligned(M, N, K, sampled, beta):
    # a bf16 C that starts 2 bytes into its allocation cannot take the paired
    # 4-byte stores: the per-value epilogue (half tiles, and whole waves)
    ah = datagen.host_input(datagen.act(tokens=M, hidden=K, seed=31))
    bh = datagen.host_input(datagen.weight(out_features=N, in_features=K, seed=32))
    qa, qb = oracle.quantize_1d(ah), oracle.quantize_1d(bh, rounding=1, seed=6)
    up = lambda q: nv.Quantized(torch.from_numpy(q[0]).to(DEV), torch.from_numpy(q[1]).to(DEV),
                                torch.from_numpy(q[2]).to(DEV))
    if sampled:
        rng = np.random.default_rng(8)
        ii = np.concatenate([[0, M - 1], rng.integers(0, M, 3000)]).astype(np.int64)
        jj = np.concatenate([[0, N - 1], rng.integers(0, N, 3000)]).astype(np.int64)
        ref, absum = oracle.gemm_sample(qa[0], qa[1], qa[2][0], qb[0], qb[1], qb[2][0], ii, jj)
    else:
        ref, absum = oracle.gemm(qa[0], qa[1], qa[2][0], qb[0], qb[1], qb[2][0])
    g = torch.Generator().manual_seed(9)
    c_in = (torch.randn(M, N, generator=g) * float(np.abs(ref).max())).to(torch.bfloat16)
    store = torch.empty(M * N + 1, dtype=torch.bfloat16, device=DEV)
    c = store[1:].view(M, N)
    assert c.data_ptr() % 4 == 2
    c.copy_(c_in.to(DEV))
    amax = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    nv.gemm_ex(up(qa), up(qb), out=c, beta=beta, amax=amax)
    torch.cuda.synchronize()
    got_all = c.float().cpu().numpy()
    cin = c_in.float().numpy().astype(np.float64)
    if sampled:
        got, cin = got_all[ii, jj].astype(np.float64), cin[ii, jj]
    else:
        got = got_all.astype(np.float64)
    want = ref + beta * cin
    bound = (1e-5 * absum + 2.0 ** -22 * (np.abs(ref) + np.abs(beta * cin))) * (1 + 2.0 ** -8) \
        + 2.0 ** -8 * np.abs(want)
    excess = np.abs(got - want) - bound
    assert excess.max() <= 0, f"max excess {excess.max()}"
    assert amax.item() == float(np.abs(got_all).max())
