"""GPU parity of the MXFP4 quantizer, dequantizer and GEMM against the oracle.

MXFP4 (OCP Microscaling Formats (MX) v1.0: 32-element blocks, E8M0 scales)
is the format "Pretraining Large Language Models with NVFP4", Technische
samenvatting 2A, compares NVFP4 with.  Quantizer codes and scale bytes must
match the oracle bit for bit; dequantized values are exact, so the fp32
output must equal the oracle's value and the bf16 output its nearest-even
rounding; GEMM results must lie within 1e-5 * sum_k |a_ik b_jk| of the
oracle's double-precision sum.  GEMM and dequantizer inputs are the oracle's
quantizations, never the GPU's."""
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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 32), (7, 96), (48, 80 * 2), (160, 288), (304, 4096), (33, 2080)])
def test_mx_quantize(shape, dtype):
    x = datagen.sweep(*shape, seed=shape[1])
    x = x.float() if dtype == "f32" else x
    q = nv.mx_quantize(x.to(DEV))
    torch.cuda.synchronize()
    codes, scales = oracle.mx_quantize(datagen.host_input(x))
    assert np.array_equal(host(q.scales), scales)
    bad = np.argwhere(host(q.codes) != codes)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[:4].tolist()}"


def test_mx_quantize_edge_values():
    x = torch.zeros(6, 64)
    x[1, :32] = -0.0
    x[2, 0], x[2, 1] = 8e-39, -3e-39            # exponent clamped to -127
    x[3, :8] = torch.tensor([7.0, 3.3, -0.2, 0.25, 0.75, 2.5, -5.0, 1.4])
    x[4, 32:] = 3.0e38                          # largest exponents
    x[5, :] = torch.linspace(-6.5, 6.5, 64)
    q = nv.mx_quantize(x.to(DEV))
    torch.cuda.synchronize()
    codes, scales = oracle.mx_quantize(x.numpy())
    assert np.array_equal(host(q.scales), scales)
    assert np.array_equal(host(q.codes), codes)


def test_mx_quantize_full_size_gradient():
    g = datagen.grad(DEV)
    q = nv.mx_quantize(g)
    torch.cuda.synchronize()
    codes, scales = oracle.mx_quantize(datagen.host_input(g))
    assert np.array_equal(host(q.scales), scales)
    assert np.array_equal(host(q.codes), codes)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mx_dequantize(dtype):
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 256, size=(253, 64), dtype=np.uint8)
    scales = np.repeat(np.arange(253, dtype=np.uint8)[:, None], 4, axis=1)  # every byte 0 .. 252
    q = nv.MxQuantized(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV))
    out = nv.mx_dequantize(q, dtype=dtype)
    torch.cuda.synchronize()
    want = torch.from_numpy(oracle.mx_dequantize(codes, scales).astype(np.float32))
    if dtype == torch.bfloat16:
        want = want.to(torch.bfloat16)
    got = out.cpu()
    iv = torch.int32 if dtype == torch.float32 else torch.int16
    assert torch.equal(got.view(iv), want.view(iv))


def check_gemm(ac, as_, bc, bs, sample=None):
    M, K = ac.shape[0], ac.shape[1] * 2
    N = bc.shape[0]
    a = nv.MxQuantized(torch.from_numpy(ac).to(DEV), torch.from_numpy(as_).to(DEV))
    b = nv.MxQuantized(torch.from_numpy(bc).to(DEV), torch.from_numpy(bs).to(DEV))
    c = nv.mx_gemm(a, b)
    torch.cuda.synchronize()
    c = host(c).astype(np.float64)
    if sample is None:
        ref, absum = oracle.mx_gemm(ac, as_, bc, bs)
        err = np.abs(c - ref)
    else:
        ii, jj = sample
        ref, absum = oracle.mx_gemm(ac, as_, bc, bs, ii, jj)
        err = np.abs(c[ii, jj] - ref)
    worst = np.max(err - 1e-5 * absum)
    assert worst <= 0, f"max excess {worst}, rel {np.max(err / (absum + 1e-300))}"


def quantized(rows, cols, seed, kind="act"):
    if kind == "act":
        t = datagen.act(tokens=rows, hidden=cols, seed=seed)
    elif kind == "weight":
        t = datagen.weight(out_features=rows, in_features=cols, seed=seed)
    else:
        t = datagen.grad(tokens=rows, out_features=cols, seed=seed)
    return oracle.mx_quantize(datagen.host_input(t))


# general path (ragged) and fast path (multiples of 256) shapes
@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (40, 24, 160), (100, 70, 96), (33, 300, 544),
                                   (256, 256, 256), (512, 256, 768), (256, 512, 512), (768, 512, 1024)])
def test_mx_gemm_small(M, N, K):
    ac, as_ = quantized(M, K, seed=M, kind="act")
    bc, bs = quantized(N, K, seed=N + 1, kind="weight")
    check_gemm(ac, as_, bc, bs)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,M,N,K,ka,kb", [
    ("fprop", 8192, 20480, 5120, "act", "weight"),
    ("dgrad", 8192, 5120, 20480, "grad", "weight"),
    ("wgrad", 20480, 5120, 8192, "grad", "act"),
])
def test_mx_gemm_full_size_sampled(name, M, N, K, ka, kb):
    ac, as_ = quantized(M, K, seed=0, kind=ka)
    bc, bs = quantized(N, K, seed=1, kind=kb)
    rng = np.random.default_rng(7)
    ii = np.concatenate([rng.integers(0, M, 2048), [0, M - 1, 255, 256]])
    jj = np.concatenate([rng.integers(0, N, 2048), [N - 1, 0, 256, 255]])
    check_gemm(ac, as_, bc, bs, sample=(ii, jj))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("K", [1 << 24, (1 << 24) + 256])
def test_mx_gemm_largest_k_either_side_of_the_fast_path_limit(K):
    """The fast MXFP4 kernel takes K up to 2^24 (32-bit operand offsets);
    2^24 + 256 goes to the general kernel.  A 256 x 256 product of random
    codes and E8M0 bytes (2 GiB per operand) against the oracle at the four
    corners and 60 random outputs."""
    M = N = 256
    g = torch.Generator(device=DEV).manual_seed(K)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=DEV, generator=g)
    bc = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=DEV, generator=g)
    as_ = torch.randint(118, 136, (M, K // 32), dtype=torch.uint8, device=DEV, generator=g)
    bs = torch.randint(118, 136, (N, K // 32), dtype=torch.uint8, device=DEV, generator=g)
    c = nv.mx_gemm(nv.MxQuantized(ac, as_), nv.MxQuantized(bc, bs))
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    ii = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, 60)]).astype(np.int64)
    jj = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 60)]).astype(np.int64)
    ref, absum = oracle.mx_gemm(ac.cpu().numpy(), as_.cpu().numpy(), bc.cpu().numpy(), bs.cpu().numpy(),
                                ii, jj)
    got = c[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= 1e-5 * absum), np.max(err / absum)
