"""The C-ABI library loads, exports every symbol include/nvfp4.h declares, and
rejects invalid arguments on the host before any HIP call (so these checks
need no GPU).  Also checks that the product path has no CPU fallback."""
import ctypes
import os
import re

import pytest
import torch

import bit_block_scaled_quant_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:nv|mx)fp4_\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("nvfp4_quantize", "nvfp4_quantize_2d", "nvfp4_quantize_cast_transpose", "nvfp4_rht",
              "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_status_string", "nvfp4_last_error",
              "mxfp4_quantize", "mxfp4_dequantize", "mxfp4_gemm", "nvfp4_gemm_ex",
              "nvfp4_quantize_with_amax"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = nv.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_status_strings():
    L = nv.lib()
    assert L.nvfp4_status_string(0) == b"ok"
    assert L.nvfp4_status_string(-2) == b"invalid shape"
    assert L.nvfp4_last_error() == b""


# fake, well-aligned device addresses: validation must fail before they are used
A16 = ctypes.c_void_p(0x10000)
A8 = ctypes.c_void_p(0x20008)


def q(x=A16, dtype=1, rows=32, cols=64, rounding=0, seed=0, rht=0, rht_seed=0, codes=A16,
      scales=A16, ts=A16, codes_t=None, scales_t=None):
    return nv.lib().nvfp4_quantize(x, dtype, rows, cols, rounding, seed, rht, rht_seed, codes,
                                   scales, ts, codes_t, scales_t, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), -1), (dict(codes=None), -1), (dict(scales=None), -1), (dict(ts=None), -1),
    (dict(dtype=2), -1), (dict(rounding=2), -1), (dict(rht=2), -1),
    (dict(codes_t=A16), -1), (dict(codes_t=A16, scales_t=A16, rht=1), -1),
    (dict(cols=24), -2), (dict(cols=0), -2), (dict(rows=0), -2), (dict(rows=-5), -2),
    (dict(rows=40, codes_t=A16, scales_t=A16), -2), (dict(rows=1 << 40, cols=1 << 10), -2),
    (dict(x=A8), -3), (dict(codes=ctypes.c_void_p(0x10004)), -3),
    (dict(ts=ctypes.c_void_p(0x10002)), -3),
    (dict(codes_t=ctypes.c_void_p(0x10004), scales_t=A16), -3),
])
def test_quantize_rejects_bad_arguments(kw, status):
    assert q(**kw) == status


def test_quantize_2d_rejects_bad_arguments():
    L = nv.lib()
    f = L.nvfp4_quantize_2d
    assert f(A16, 1, 40, 64, 0, 0, A16, A16, A16, None, None, None) == -2  # rows % 16
    assert f(A16, 1, 32, 40, 0, 0, A16, A16, A16, None, None, None) == -2  # cols % 16
    assert f(A16, 3, 32, 64, 0, 0, A16, A16, A16, None, None, None) == -1
    assert f(A16, 1, 32, 64, 0, 0, A16, A16, A16, A16, None, None) == -1
    assert f(A8, 1, 32, 64, 0, 0, A16, A16, A16, None, None, None) == -3


def test_cast_transpose_rejects_bad_arguments():
    f = nv.lib().nvfp4_quantize_cast_transpose

    def ct(x=A16, dtype=1, rows=32, cols=64, rounding=0, rht_t=1, codes=A16, scales=A16, ts=A16,
           codes_t=A16, scales_t=A16, ts_t=A16):
        return f(x, dtype, rows, cols, rounding, 0, 1, rht_t, 0, codes, scales, ts, codes_t, scales_t,
                 ts_t, None)
    assert ct(codes_t=None) == -1
    assert ct(scales_t=None) == -1
    assert ct(ts_t=None) == -1
    assert ct(x=None) == -1
    assert ct(rht_t=2) == -1
    assert ct(rounding=3) == -1
    assert ct(rows=40) == -2   # rows % 16
    assert ct(cols=40) == -2   # cols % 16
    assert ct(rows=0) == -2
    assert ct(x=A8) == -3
    assert ct(ts_t=ctypes.c_void_p(0x10002)) == -3
    assert ct(codes_t=ctypes.c_void_p(0x10004)) == -3


def test_dequantize_rejects_bad_arguments():
    f = nv.lib().nvfp4_dequantize
    assert f(None, A16, A16, 16, 32, 0, A16, None) == -1
    assert f(A16, A16, A16, 16, 32, 2, A16, None) == -1   # out dtype
    assert f(A16, A16, A16, 16, 24, 0, A16, None) == -2   # cols % 16
    assert f(A16, A16, A16, 0, 32, 0, A16, None) == -2
    assert f(A16, A16, A16, 16, 32, 0, A8, None) == -3    # out alignment
    assert f(ctypes.c_void_p(0x10004), A16, A16, 16, 32, 0, A16, None) == -3


def test_mx_calls_reject_bad_arguments():
    L = nv.lib()
    assert L.mxfp4_quantize(A16, 1, 4, 48, A16, A16, None) == -2   # cols % 32
    assert L.mxfp4_quantize(A16, 2, 4, 64, A16, A16, None) == -1
    assert L.mxfp4_quantize(None, 1, 4, 64, A16, A16, None) == -1
    assert L.mxfp4_quantize(A8, 1, 4, 64, A16, A16, None) == -3
    assert L.mxfp4_dequantize(A16, A16, 4, 48, 0, A16, None) == -2
    assert L.mxfp4_dequantize(A16, A16, 4, 64, 0, A8, None) == -3
    g = L.mxfp4_gemm
    assert g(A16, A16, A16, A16, 16, 16, 48, A16, None) == -2   # K % 32
    assert g(A16, A16, A16, A16, 0, 16, 64, A16, None) == -2
    assert g(None, A16, A16, A16, 16, 16, 64, A16, None) == -1
    assert g(A8, A16, A16, A16, 16, 16, 64, A16, None) == -3    # codes 16-byte aligned
    assert g(A16, A16, A16, A16, 65535 * 64 + 64, 16, 64, A16, None) == -2   # M above the grid limit
    assert g(A16, A16, A16, A16, 1 << 21, 16, 1 << 20, A16, None) == -2      # M * K above 2^40


def test_gemm_ex_and_quantize_with_amax_reject_bad_arguments():
    L = nv.lib()
    g = L.nvfp4_gemm_ex
    F = ctypes.c_float
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 32, A16, 2, F(0.0), None, None) == -1   # C dtype
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 32, A16, 0, F(float("nan")), None, None) == -1
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 32, A16, 0, F(float("inf")), None, None) == -1
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 24, A16, 0, F(0.0), None, None) == -2
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 32, ctypes.c_void_p(0x10002), 0, F(0.0), None, None) == -3
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 32, A16, 0, F(0.0), ctypes.c_void_p(0x10002), None) == -3
    q = L.nvfp4_quantize_with_amax
    assert q(A16, 1, 4, 24, 0, 0, 0, 0, A16, A16, A16, None) == -2
    assert q(A16, 1, 4, 32, 0, 0, 2, 0, A16, A16, A16, None) == -1
    assert q(None, 1, 4, 32, 0, 0, 0, 0, A16, A16, A16, None) == -1


def test_rht_and_gemm_reject_bad_arguments():
    L = nv.lib()
    assert L.nvfp4_rht(A16, 1, 4, 24, 0, A16, None) == -2
    assert L.nvfp4_rht(None, 1, 4, 32, 0, A16, None) == -1
    assert L.nvfp4_rht(A16, 1, 4, 32, 0, A8, None) == -3
    g = L.nvfp4_gemm
    assert g(A16, A16, A16, A16, A16, A16, 16, 16, 24, A16, None) == -2
    assert g(A16, A16, A16, A16, A16, A16, 0, 16, 32, A16, None) == -2
    assert g(None, A16, A16, A16, A16, A16, 16, 16, 32, A16, None) == -1
    assert g(ctypes.c_void_p(0x10004), A16, A16, A16, A16, A16, 16, 16, 32, A16, None) == -3
    assert g(A16, A16, A16, A16, A16, A16, 65535 * 128 + 16, 16, 32, A16, None) == -2  # M above the grid limit
    assert g(A16, A16, A16, A16, A16, A16, 1 << 21, 16, 1 << 20, A16, None) == -2      # M * K above 2^40
    assert g(A16, A16, A16, A16, A16, A16, 16, 1 << 21, 1 << 20, A16, None) == -2      # N * K above 2^40
    assert g(A16, A16, A16, A16, A16, A16, 1 << 20, 1 << 21, 16, A16, None) == -2      # M * N above 2^40


def test_no_cpu_fallback():
    x = torch.zeros(16, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv.quantize(x)
