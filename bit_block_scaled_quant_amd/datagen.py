"""Seeded synthetic inputs shaped like the linear layers of a 12B-class
hybrid Mamba-Transformer (the workload of "Pretraining Large Language Models
with NVFP4", section 3 "Belangrijkste Resultaten").

This module holds no part of the quantizer or GEMM arithmetic: it only draws
tensors.  Both the HIP path and the CPU oracle consume the same bytes.  Every
tensor has its own torch generator seeded from (seed, tag), so a tensor does
not depend on which others were drawn before it.  Values drawn on a GPU differ
from values drawn on the CPU for the same seed; nothing relies on them being
equal, because each check hands the very same bytes to both sides.

Recipes (shapes are parameters so tests can shrink them):
  tiny      A, B [256 x 256] fp32 ~ N(0,1); 1% of entries (655 of 65536,
            chosen by a seeded permutation) multiplied by 50.
  act       X [tokens x hidden] bf16 ~ N(0,1); 0.1% of the columns (5 of
            5120) multiplied by 30 (outlier channels).
  weight    W [out x in] bf16 ~ N(0, 0.02^2).
  grad      dY [tokens x out] bf16 = 1e-3 * z + 1e-3 * t3 with z ~ N(0,1) and
            t3 = z0 / sqrt((z1^2 + z2^2 + z3^2) / 3) a Student-t(3) variate.
  sweep     bf16 ~ N(0,1); 0.1% of the entries multiplied by 100.
bf16 tensors are drawn in fp32 and cast with round-to-nearest-even.
"""
import torch

TAG_A, TAG_B, TAG_X, TAG_W, TAG_DY, TAG_SWEEP = 1, 2, 3, 4, 5, 6


def _gen(device, seed, tag):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1009 + int(tag))
    return g


def tiny(device="cpu", seed=0, rows=256, cols=256, tag=TAG_A):
    g = _gen(device, seed, tag)
    x = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    n = rows * cols
    k = int(round(0.01 * n))
    idx = torch.randperm(n, generator=g, device=device)[:k]
    x.view(-1)[idx] *= 50.0
    return x


def act(device="cpu", seed=0, tokens=8192, hidden=5120, outlier_frac=0.001, outlier_mult=30.0):
    g = _gen(device, seed, TAG_X)
    x = torch.randn(tokens, hidden, generator=g, device=device, dtype=torch.float32)
    k = max(1, int(round(outlier_frac * hidden)))
    cols = torch.randperm(hidden, generator=g, device=device)[:k]
    x[:, cols] *= outlier_mult
    return x.to(torch.bfloat16)


def weight(device="cpu", seed=0, out_features=20480, in_features=5120, std=0.02):
    g = _gen(device, seed, TAG_W)
    w = torch.randn(out_features, in_features, generator=g, device=device, dtype=torch.float32)
    return (w * std).to(torch.bfloat16)


def grad(device="cpu", seed=0, tokens=8192, out_features=20480, sigma=1e-3):
    g = _gen(device, seed, TAG_DY)
    shape = (tokens, out_features)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    z0 = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(3):
        zi = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi += zi * zi
    t3 = z0 / torch.sqrt(chi / 3.0)
    del chi
    return (sigma * z + sigma * t3).to(torch.bfloat16)


def sweep(rows, cols, device="cpu", seed=0, outlier_frac=0.001, outlier_mult=100.0):
    g = _gen(device, seed, TAG_SWEEP + 7 * rows + cols)
    x = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    n = rows * cols
    k = max(1, int(round(outlier_frac * n)))
    idx = torch.randperm(n, generator=g, device=device)[:k]
    x.view(-1)[idx] *= outlier_mult
    return x.to(torch.bfloat16)


def bf16_bits(t):
    """numpy uint16 view of a bf16 tensor's bit patterns (host copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


def host_input(t):
    """numpy array the oracle accepts: float32, or uint16 bf16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    assert t.dtype == torch.float32
    return t.detach().contiguous().cpu().numpy()
