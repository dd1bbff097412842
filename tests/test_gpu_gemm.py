"""GPU parity of the block-scaled GEMM against the oracle.

Operands are quantized by the oracle (never by the HIP path) from the seeded
workload tensors, uploaded, multiplied on the GPU, and every output (small
cases) or a sample of outputs that covers the edges and every tile position
(full-size cases) must satisfy |C_gpu - C| <= 1e-5 * sum_k |a_ik b_jk| with C
and the sum computed by the oracle in double."""
import numpy as np
import pytest
import torch

import bit_block_scaled_quant_amd as nv
import oracle
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-5


def upload(ref):
    codes, scales, ts = ref[0], ref[1], ref[2]
    return nv.Quantized(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                        torch.from_numpy(ts).to(DEV))


def check_full(c_gpu, ref, refabs):
    c = c_gpu.detach().cpu().numpy().astype(np.float64)
    err = np.abs(c - ref)
    bad = np.argwhere(err > TOL * refabs)
    assert bad.size == 0, (f"{len(bad)} outputs outside tolerance, first {bad[:4].tolist()}, "
                           f"worst ratio {np.max(err / np.maximum(refabs, 1e-300))}")
    return float(np.max(err / np.maximum(refabs, 1e-300)))


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (64, 64, 128), (200, 136, 272),
                                   (130, 250, 512), (1, 1, 16), (17, 300, 48), (129, 129, 1024),
                                   (384, 128, 4096), (256, 256, 512), (512, 768, 1024),
                                   (768, 256, 3072), (256, 256, 64), (512, 256, 448),
                                   (256, 512, 320)])
def test_gemm_small(M, N, K):
    a = datagen.tiny(tag=datagen.TAG_A, rows=M, cols=K, seed=M)
    b = datagen.tiny(tag=datagen.TAG_B, rows=N, cols=K, seed=N)
    ra = oracle.quantize_1d(a.numpy())
    rb = oracle.quantize_1d(b.numpy(), rounding=1, seed=3)
    c = nv.gemm(upload(ra), upload(rb))
    torch.cuda.synchronize()
    ref, refabs = oracle.gemm(ra[0], ra[1], ra[2][0], rb[0], rb[1], rb[2][0])
    check_full(c, ref, refabs)


def test_gemm_random_codes_and_scales():
    rng = np.random.default_rng(0)
    M, N, K = 256, 512, 1536
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    asc = rng.integers(0, 0x7F, (M, K // 16), dtype=np.uint8)
    bsc = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    ta, tb = np.array([0.37, 1.0], np.float32), np.array([1234.5, 1.0], np.float32)
    c = nv.gemm(upload((ac, asc, ta)), upload((bc, bsc, tb)))
    torch.cuda.synchronize()
    ref, refabs = oracle.gemm(ac, asc, ta[0], bc, bsc, tb[0])
    check_full(c, ref, refabs)


@pytest.mark.parametrize("M,N,K", [(256, 192, 2048), (512, 256, 2048)])
def test_gemm_exact_with_unit_scales(M, N, K):
    """Scale bytes 0x38 (1.0) and S = 1: every partial sum is a multiple of
    0.25 below 2^22, so the fp32 result must be exact."""
    rng = np.random.default_rng(1)
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ones = lambda r: np.full((r, K // 16), 0x38, np.uint8)
    t1 = np.array([1.0, 2688.0], np.float32)
    c = nv.gemm(upload((ac, ones(M), t1)), upload((bc, ones(N), t1)))
    torch.cuda.synchronize()
    ref, _ = oracle.gemm(ac, ones(M), 1.0, bc, ones(N), 1.0)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("M,N,K", [(256, 256, 512), (100, 70, 96)])
@pytest.mark.parametrize("sa,sb", [(1e-30, 1e30), (1e30, 1e-30)])
def test_gemm_extreme_tensor_scales(M, N, K, sa, sb):
    # tensor scales near 2.7e33 and 2.7e-27: the reciprocals are applied one
    # after the other in fp32, and every intermediate stays a normal number
    a = datagen.tiny(tag=datagen.TAG_A, rows=M, cols=K, seed=7) * sa
    b = datagen.tiny(tag=datagen.TAG_B, rows=N, cols=K, seed=8) * sb
    ra = oracle.quantize_1d(a.numpy())
    rb = oracle.quantize_1d(b.numpy(), rounding=1, seed=4)
    c = nv.gemm(upload(ra), upload(rb))
    torch.cuda.synchronize()
    ref, refabs = oracle.gemm(ra[0], ra[1], ra[2][0], rb[0], rb[1], rb[2][0])
    assert np.abs(ref).max() > 1.0  # the product itself is of ordinary size
    check_full(c, ref, refabs)


def test_gemm_symmetry_and_determinism():
    a = datagen.tiny(tag=datagen.TAG_A, rows=192, cols=512, seed=5)
    b = datagen.tiny(tag=datagen.TAG_B, rows=320, cols=512, seed=6)
    qa, qb = upload(oracle.quantize_1d(a.numpy())), upload(oracle.quantize_1d(b.numpy()))
    c1 = nv.gemm(qa, qb)
    c2 = nv.gemm(qa, qb)
    ct = nv.gemm(qb, qa)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2)
    assert torch.allclose(c1, ct.t(), rtol=1e-6, atol=0)


def sample_positions(M, N, n=3000, seed=0):
    rng = np.random.default_rng(seed)
    # complete first and last rows and columns
    ii = [np.zeros(N, np.int64), np.full(N, M - 1, np.int64), np.arange(M), np.arange(M)]
    jj = [np.arange(N), np.arange(N), np.zeros(M, np.int64), np.full(M, N - 1, np.int64)]
    # every position inside a 256 x 256 tile at least once (row t % 256 with a
    # random tile, column t % 256 with a random tile), and random outputs
    t = np.arange(256)
    ii += [(t + 256 * rng.integers(0, max(1, M // 256), 256)) % M, rng.integers(0, M, 256)]
    jj += [rng.integers(0, N, 256), (t + 256 * rng.integers(0, max(1, N // 256), 256)) % N]
    ii.append(rng.integers(0, M, n))
    jj.append(rng.integers(0, N, n))
    # one output in every 256 x 128 block (a whole tile is two, a half tile one)
    bi, bj = [], []
    for bm in range(0, M, 256):
        for bn in range(0, N, 128):
            bi.append(bm + int(rng.integers(0, min(256, M - bm))))
            bj.append(bn + int(rng.integers(0, min(128, N - bn))))
    ii.append(np.array(bi, np.int64))
    jj.append(np.array(bj, np.int64))
    return np.concatenate(ii).astype(np.int64), np.concatenate(jj).astype(np.int64)


def check_every_output(c_gpu, a_ref, b_ref):
    """Every output against the oracle's dense form (its per-element
    dequantization contracted in float64); returns the largest
    |err| / sum |ab|."""
    ref, refabs = oracle.gemm_dense(a_ref[0], a_ref[1], a_ref[2][0], b_ref[0], b_ref[1], b_ref[2][0])
    got = c_gpu.cpu().numpy()
    worst = 0.0
    for r0 in range(0, got.shape[0], 1024):  # compared a band of rows at a time
        err = np.abs(got[r0:r0 + 1024].astype(np.float64) - ref[r0:r0 + 1024])
        bound = TOL * refabs[r0:r0 + 1024]
        bad = np.argwhere(err > bound)
        assert bad.size == 0, (f"{len(bad)} outputs outside tolerance in rows {r0}.., first "
                               f"{(bad[:4] + [r0, 0]).tolist()}")
        worst = max(worst, float(np.max(err / np.maximum(refabs[r0:r0 + 1024], 1e-300))))
    return worst


def gemm_full_case(a_ref, b_ref, M, N, K):
    # C starts as NaN, so the finiteness check below also shows every output was written
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    nv.gemm(upload(a_ref), upload(b_ref), out=c)
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    # the oracle's own double sums at complete first / last rows and columns,
    # every tile position and random outputs ...
    ii, jj = sample_positions(M, N)
    ref, refabs = oracle.gemm_sample(a_ref[0], a_ref[1], a_ref[2][0], b_ref[0], b_ref[1],
                                     b_ref[2][0], ii, jj)
    got = c[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)].cpu().numpy()
    err = np.abs(got.astype(np.float64) - ref)
    assert np.all(err <= TOL * refabs), np.max(err / np.maximum(refabs, 1e-300))
    # ... and every output against the dense form
    worst = check_every_output(c, a_ref, b_ref)
    print(f"gemm {M}x{N}x{K}: {M * N} outputs, worst |err| / sum|ab| = {worst:.3g}", flush=True)


@pytest.mark.timeout(900)
def test_gemm_full_fprop():
    x = datagen.act(DEV)
    w = datagen.weight(DEV)
    gemm_full_case(oracle.quantize_1d(datagen.bf16_bits(x)),
                   oracle.quantize_2d(datagen.bf16_bits(w), transposed=False), 8192, 20480, 5120)


@pytest.mark.timeout(900)
def test_gemm_full_dgrad():
    dy = datagen.grad(DEV)
    w = datagen.weight(DEV)
    qw = oracle.quantize_2d(datagen.bf16_bits(w))
    gemm_full_case(oracle.quantize_1d(datagen.bf16_bits(dy), rounding=1),
                   (qw[3], qw[4], qw[2]), 8192, 5120, 20480)


@pytest.mark.timeout(900)
def test_gemm_full_wgrad():
    dyt = datagen.grad(DEV).t().contiguous()
    xt = datagen.act(DEV).t().contiguous()
    gemm_full_case(oracle.quantize_1d(datagen.bf16_bits(dyt), rounding=1, rht=1),
                   oracle.quantize_1d(datagen.bf16_bits(xt), rht=1), 20480, 5120, 8192)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N", [(8448, 2816), (4096, 4352), (4096, 4608)])
def test_gemm_ragged_tile_counts(M, N):
    # 363 tiles (XCD runs of unequal length, idle workgroups in the last one),
    # 272 tiles (a last wave of 256 x 128 halves) and 288 tiles (a last wave
    # of 256 x 64 quarters after a whole one); sampled outputs against the
    # oracle, every output written
    K = 512
    a = datagen.host_input(datagen.act(tokens=M, hidden=K, seed=M))
    b = datagen.host_input(datagen.weight(out_features=N, in_features=K, seed=N))
    gemm_full_case(oracle.quantize_1d(a), oracle.quantize_1d(b, rounding=1, seed=2), M, N, K)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N,K", [(8192, 20480, 5120), (8192, 5120, 20480), (20480, 5120, 8192),
                                   (8448, 2816, 512)])
def test_gemm_plain_and_ex_epilogues_agree(M, N, K):
    # nvfp4_gemm and nvfp4_gemm_ex (fp32 out, beta 0, with an amax target)
    # run the same MFMA sequence per output with different epilogue code:
    # the outputs must agree bit for bit everywhere, and the amax is max |C|
    a = nv.quantize(datagen.act(tokens=M, hidden=K, seed=1).to(DEV))
    b = nv.quantize(datagen.weight(out_features=N, in_features=K, seed=2).to(DEV), rounding=1, seed=3)
    c1 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    nv.gemm(a, b, out=c1)
    c2 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    amax = torch.zeros(1, dtype=torch.float32, device=DEV)
    nv.gemm_ex(a, b, out=c2, amax=amax)
    torch.cuda.synchronize()
    assert torch.isfinite(c1).all()
    assert torch.equal(c1, c2)
    assert amax.item() == c1.abs().max().item()


def test_tiny_config_as_stated():
    """The Tiny workload as stated: A, B [256 x 256] fp32 N(0,1) with 1% of the
    entries x50, seed 0; both quantized 1D with RNE by the HIP path; their
    codes, scale bytes and tensor scales equal the oracle's bit for bit; the
    HIP GEMM of those operands matches the oracle at all 65,536 outputs."""
    a = datagen.tiny(seed=0, tag=datagen.TAG_A)
    b = datagen.tiny(seed=0, tag=datagen.TAG_B)
    qa, qb = nv.quantize(a.to(DEV)), nv.quantize(b.to(DEV))
    c = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    ra, rb = oracle.quantize_1d(a.numpy()), oracle.quantize_1d(b.numpy())
    for got, want in ((qa.codes, ra[0]), (qa.scales, ra[1]), (qa.tensor_scale, ra[2]),
                      (qb.codes, rb[0]), (qb.scales, rb[1]), (qb.tensor_scale, rb[2])):
        assert np.array_equal(got.cpu().numpy(), want)
    ref, refabs = oracle.gemm(ra[0], ra[1], ra[2][0], rb[0], rb[1], rb[2][0])
    assert c.shape == (256, 256)
    check_full(c, ref, refabs)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("K", [512, 1024])
def test_gemm_whole_wave_complete_output(K):
    """4096 x 4096 is 256 whole 256 x 256 tiles, one full wave of the fast
    kernel on 256 CUs: every one of the 16.8M outputs against the oracle."""
    M = N = 4096
    a = datagen.host_input(datagen.act(tokens=M, hidden=K, seed=3))
    b = datagen.host_input(datagen.weight(out_features=N, in_features=K, seed=4))
    ra, rb = oracle.quantize_1d(a), oracle.quantize_1d(b, rounding=1, seed=5)
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    nv.gemm(upload(ra), upload(rb), out=c)
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    worst = check_every_output(c, ra, rb)
    print(f"whole wave K={K}: worst |err| / sum|ab| = {worst:.3g}", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N", [(4096, 4096), (256, 512)])
def test_gemm_same_sign_large_k(M, N):
    """No cancellation at the largest K of the workload (20480): every
    product is non-negative, so every partial sum grows and the fp32
    accumulation error is as large relative to sum |ab| as data makes it.
    4096 x 4096 runs the whole-tile kernel, 256 x 512 the half-tile one;
    every output must stay within 1e-5 * sum |ab| (the worst ratio is
    printed)."""
    K = 20480
    a = datagen.act(tokens=M, hidden=K, seed=6).float().abs()
    b = datagen.weight(out_features=N, in_features=K, seed=7).float().abs()
    ra = oracle.quantize_1d(a.numpy())
    rb = oracle.quantize_1d(b.numpy())
    c = nv.gemm(upload(ra), upload(rb))
    torch.cuda.synchronize()
    worst = check_every_output(c, ra, rb)
    print(f"same sign {M}x{N}x{K}: worst |err| / sum|ab| = {worst:.3g}", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("K", [1 << 24, (1 << 24) + 512])
def test_gemm_largest_k_either_side_of_the_fast_path_limit(K):
    """The whole-tile kernel forms operand offsets in 32 bits and takes K up
    to 2^24; one step more goes to the general kernel, whose offsets are 64
    bit.  A 256 x 256 product at K = 2^24 and 2^24 + 512 (random codes and
    scale bytes, 2 GiB per operand) against the oracle's double sums at the
    four corners and 60 random outputs."""
    M = N = 256
    g = torch.Generator(device=DEV).manual_seed(K)
    ac = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=DEV, generator=g)
    bc = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=DEV, generator=g)
    asc = torch.randint(0x28, 0x48, (M, K // 16), dtype=torch.uint8, device=DEV, generator=g)
    bsc = torch.randint(0x28, 0x48, (N, K // 16), dtype=torch.uint8, device=DEV, generator=g)
    ta = torch.tensor([3.0, 1.0], device=DEV)
    tb = torch.tensor([0.75, 1.0], device=DEV)
    c = nv.gemm(nv.Quantized(ac, asc, ta), nv.Quantized(bc, bsc, tb))
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    ii = np.concatenate([[0, 0, M - 1, M - 1], rng.integers(0, M, 60)]).astype(np.int64)
    jj = np.concatenate([[0, N - 1, 0, N - 1], rng.integers(0, N, 60)]).astype(np.int64)
    ref, refabs = oracle.gemm_sample(ac.cpu().numpy(), asc.cpu().numpy(), 3.0, bc.cpu().numpy(),
                                     bsc.cpu().numpy(), 0.75, ii, jj)
    got = c[torch.from_numpy(ii).to(DEV), torch.from_numpy(jj).to(DEV)].cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    assert np.all(err <= TOL * refabs), np.max(err / refabs)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("M,N,K", [(4000, 5008, 1040), (4452, 3600, 528)])
def test_gemm_general_path_large_ragged(M, N, K):
    """Shapes off the whole-tile kernel's grid with enough 256 x 256 tiles
    to fill the chip (16 x 20 and 18 x 15, ragged at the bottom and right),
    so the general kernel runs its large tiles, with K not a multiple of its
    128-element step: every output against the oracle's dense form."""
    a = datagen.host_input(datagen.act(tokens=M, hidden=K, seed=K))
    b = datagen.host_input(datagen.weight(out_features=N, in_features=K, seed=N))
    ra, rb = oracle.quantize_1d(a), oracle.quantize_1d(b, rounding=1, seed=4)
    c = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    nv.gemm(upload(ra), upload(rb), out=c)
    torch.cuda.synchronize()
    assert torch.isfinite(c).all()
    check_every_output(c, ra, rb)
