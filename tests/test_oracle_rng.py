"""Pins of the oracle's random bits.

Philox4x32-10 (Salmon et al., SC'11) against PyTorch's own header-only
implementation (ATen/core/PhiloxRNGEngine.h), compiled here with g++; plus
statistical sanity of the 16-bit stream the stochastic rounding consumes.
"""
import os
import subprocess
import sysconfig

import numpy as np
import pytest
import torch

HERE = os.path.dirname(__file__)


@pytest.fixture(scope="module")
def torch_philox(tmp_path_factory):
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    exe = str(tmp_path_factory.mktemp("ph") / "torch_philox")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc,
                    os.path.join(HERE, "helpers", "torch_philox.cpp"), "-o", exe], check=True)

    def run(triples):
        inp = "".join(f"{s} {u} {o}\n" for s, u, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w) for w in ln.split()] for ln in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


def test_philox_matches_torch(orc, torch_philox):
    rng = np.random.default_rng(5)
    triples = [(0, 0, 0), (0, 1, 0), (0, 2, 0), (1, 0, 0), (2**64 - 1, 2**32 - 1, 2**64 - 1),
               (0x0123456789ABCDEF, 2, 7)]
    for _ in range(200):
        triples.append((int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                        int(rng.integers(0, 2**32)), int(rng.integers(0, 2**63))))
    want = torch_philox(triples)
    for (seed, sub, off), w in zip(triples, want):
        ctr = [off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [seed & 0xFFFFFFFF, seed >> 32]
        got = orc.philox4x32_10(ctr, key)
        assert np.array_equal(got.astype(np.uint64), w), (seed, sub, off)


def test_sr_bits_layout_matches_torch(orc, torch_philox):
    # element i draws 16-bit half (i & 1) of word (i & 7) >> 1 of the block
    # g = i >> 3, counter (g lo, g hi, stream, 0)
    seed, stream = 0xDEADBEEF12345678, 1
    first = (1 << 35) - 40
    n = 96
    bits = orc.sr_bits_n(seed, stream, first, n)
    groups = sorted({(first + t) >> 3 for t in range(n)})
    words = dict(zip(groups, torch_philox([(seed, stream, g) for g in groups])))
    for t in range(n):
        i = first + t
        w = int(words[i >> 3][(i & 7) >> 1])
        assert bits[t] == ((w >> 16) if (i & 1) else (w & 0xFFFF))
        assert bits[t] == orc.sr_bits(seed, stream, i)


def test_rht_sign_mask_matches_torch(orc, torch_philox):
    for seed in (0, 1, 12345, 2**64 - 1):
        w = torch_philox([(seed, 2, 0)])[0]
        assert orc.rht_sign_mask(seed) == int(w[0]) & 0xFFFF


def test_sr_bits_uniform_and_uncorrelated(orc):
    n = 1 << 22
    u = orc.sr_bits_n(0, 0, 0, n).astype(np.int64)
    # chi-square over the 256 values of the high byte; 255 dof, 5 sigma bound
    counts = np.bincount(u >> 8, minlength=256)
    exp = n / 256
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert abs(chi2 - 255) < 5 * np.sqrt(2 * 255)
    # lag-1 correlation and mean
    x = (u - 32767.5) / 65536
    r = np.dot(x[:-1], x[1:]) / np.dot(x, x)
    assert abs(r) < 5 / np.sqrt(n)
    assert abs(u.mean() - 32767.5) < 5 * 65536 / np.sqrt(12 * n)


def test_sr_bits_seed_and_stream_change_bits(orc):
    a = orc.sr_bits_n(0, 0, 0, 4096)
    assert np.array_equal(a, orc.sr_bits_n(0, 0, 0, 4096))
    assert np.mean(a == orc.sr_bits_n(1, 0, 0, 4096)) < 0.01
    assert np.mean(a == orc.sr_bits_n(0, 1, 0, 4096)) < 0.01
