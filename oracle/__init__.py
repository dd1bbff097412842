"""CPU reference ("the oracle") for the NVFP4 quantizer and block-scaled GEMM
(and for MXFP4, the 32-element power-of-two-scaled format they are compared
against).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may use it; the product path never does.  The C
source (``nvfp4_oracle.c``) states every step and the passage it follows;
this module only marshals numpy arrays into it through ctypes.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")
# a separately built copy of the oracle to load instead (the mutation test
# runs the pins against deliberately broken copies this way); never rebuilt
_LIB_OVERRIDE = os.environ.get("NVFP4_ORACLE_LIB")
_lib = None

F32, BF16 = 0, 1
RNE, SR = 0, 1


def build(src=_SRC, out=_LIB_PATH):
    """Compile the oracle with gcc: IEEE binary32 steps, no FMA contraction."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB_PATH
        if not _LIB_OVERRIDE and not os.path.exists(path):
            build()
        L = ctypes.CDLL(path)
        P, I64, U64, I, F = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                             ctypes.c_int, ctypes.c_float)
        L.orc_e2m1_value.restype = ctypes.c_double
        L.orc_e2m1_value.argtypes = [I]
        L.orc_e4m3_value.restype = ctypes.c_double
        L.orc_e4m3_value.argtypes = [I]
        L.orc_e4m3_encode.restype = I
        L.orc_e4m3_encode.argtypes = [F]
        L.orc_e2m1_encode_rne.restype = I
        L.orc_e2m1_encode_rne.argtypes = [F]
        L.orc_e2m1_encode_sr.restype = I
        L.orc_e2m1_encode_sr.argtypes = [F, ctypes.c_uint32]
        L.orc_philox4x32_10.restype = None
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_sr_bits.restype = ctypes.c_uint32
        L.orc_sr_bits.argtypes = [U64, ctypes.c_uint32, U64]
        L.orc_rht_sign_mask.restype = ctypes.c_uint32
        L.orc_rht_sign_mask.argtypes = [U64]
        L.orc_rht.restype = I
        L.orc_rht.argtypes = [P, I, I64, I64, U64, P]
        L.orc_tensor_scale.restype = F
        L.orc_tensor_scale.argtypes = [F]
        L.orc_quantize_1d.restype = I
        L.orc_quantize_1d.argtypes = [P, I, I64, I64, I, U64, I, U64, P, P, P, P, P]
        L.orc_quantize_2d.restype = I
        L.orc_quantize_2d.argtypes = [P, I, I64, I64, I, U64, P, P, P, P, P]
        L.orc_dequantize.restype = I
        L.orc_dequantize.argtypes = [P, P, F, I64, I64, P]
        L.orc_gemm.restype = I
        L.orc_gemm.argtypes = [P, P, F, P, P, F, I64, I64, I64, P, P]
        L.orc_gemm_sample.restype = I
        L.orc_gemm_sample.argtypes = [P, P, F, P, P, F, I64, I64, I64, P, P, I64, P, P]
        L.orc_e4m3_encode_n.restype = I
        L.orc_e4m3_encode_n.argtypes = [P, I64, P]
        L.orc_e2m1_encode_rne_n.restype = I
        L.orc_e2m1_encode_rne_n.argtypes = [P, I64, P]
        L.orc_e2m1_encode_sr_n.restype = I
        L.orc_e2m1_encode_sr_n.argtypes = [P, P, I64, P]
        L.orc_sr_bits_n.restype = I
        L.orc_sr_bits_n.argtypes = [U64, ctypes.c_uint32, U64, I64, P]
        L.orc_num_threads.restype = I
        L.orc_num_threads.argtypes = []
        L.orc_mx_quantize.restype = I
        L.orc_mx_quantize.argtypes = [P, I, I64, I64, P, P]
        L.orc_e8m0_value.restype = ctypes.c_double
        L.orc_e8m0_value.argtypes = [I]
        L.orc_mx_dequantize.restype = I
        L.orc_mx_dequantize.argtypes = [P, P, I64, I64, P]
        L.orc_mx_gemm.restype = I
        L.orc_mx_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P, P]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle status {rc}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _input(x):
    """numpy float32 array, or uint16 array holding bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError("oracle input must be float32 or uint16 (bf16 bits)")


# --- codecs ------------------------------------------------------------
def e2m1_value(code):
    return lib().orc_e2m1_value(int(code))


def e4m3_value(byte):
    return lib().orc_e4m3_value(int(byte))


def e4m3_encode(s):
    return lib().orc_e4m3_encode(float(s))


def e2m1_encode_rne(y):
    return lib().orc_e2m1_encode_rne(float(y))


def e2m1_encode_sr(y, u16):
    return lib().orc_e2m1_encode_sr(float(y), int(u16))


def e4m3_encode_n(s):
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, dtype=np.uint8)
    _check(lib().orc_e4m3_encode_n(_ptr(s), s.size, _ptr(out)), "e4m3_encode_n")
    return out


def e2m1_encode_rne_n(y):
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    _check(lib().orc_e2m1_encode_rne_n(_ptr(y), y.size, _ptr(out)), "e2m1_encode_rne_n")
    return out


def e2m1_encode_sr_n(y, u):
    y = np.ascontiguousarray(y, dtype=np.float32)
    u = np.ascontiguousarray(u, dtype=np.uint16)
    assert u.shape == y.shape
    out = np.empty(y.shape, dtype=np.uint8)
    _check(lib().orc_e2m1_encode_sr_n(_ptr(y), _ptr(u), y.size, _ptr(out)), "e2m1_encode_sr_n")
    return out


def tensor_scale(amax):
    return lib().orc_tensor_scale(float(amax))


# --- random bits -------------------------------------------------------
def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits(seed, stream, index):
    return lib().orc_sr_bits(int(seed), int(stream), int(index))


def sr_bits_n(seed, stream, first, n):
    out = np.empty(n, dtype=np.uint16)
    _check(lib().orc_sr_bits_n(int(seed), int(stream), int(first), int(n), _ptr(out)), "sr_bits_n")
    return out


def rht_sign_mask(rht_seed):
    return lib().orc_rht_sign_mask(int(rht_seed))


# --- transform, quantizers ---------------------------------------------
def rht(x, rht_seed):
    x, dt = _input(x)
    rows, cols = x.shape
    y = np.empty((rows, cols), dtype=np.float32)
    _check(lib().orc_rht(_ptr(x), dt, rows, cols, int(rht_seed), _ptr(y)), "rht")
    return y


def quantize_1d(x, rounding=RNE, seed=0, rht=0, rht_seed=0, transposed=False):
    """Returns (codes, scales, tensor_scale[2], codes_t, scales_t)."""
    x, dt = _input(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    ts = np.zeros(2, dtype=np.float32)
    codes_t = scales_t = None
    if transposed:
        codes_t = np.zeros((cols, rows // 2), dtype=np.uint8)
        scales_t = np.zeros((cols, rows // 16), dtype=np.uint8)
    _check(lib().orc_quantize_1d(_ptr(x), dt, rows, cols, int(rounding), int(seed), int(rht),
                                 int(rht_seed), _ptr(codes), _ptr(scales), _ptr(ts),
                                 _ptr(codes_t), _ptr(scales_t)), "quantize_1d")
    return codes, scales, ts, codes_t, scales_t


def quantize_2d(w, rounding=RNE, seed=0, transposed=True):
    """Returns (codes, scales, tensor_scale[2], codes_t, scales_t)."""
    w, dt = _input(w)
    rows, cols = w.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    ts = np.zeros(2, dtype=np.float32)
    codes_t = scales_t = None
    if transposed:
        codes_t = np.zeros((cols, rows // 2), dtype=np.uint8)
        scales_t = np.zeros((cols, rows // 16), dtype=np.uint8)
    _check(lib().orc_quantize_2d(_ptr(w), dt, rows, cols, int(rounding), int(seed), _ptr(codes),
                                 _ptr(scales), _ptr(ts), _ptr(codes_t), _ptr(scales_t)),
           "quantize_2d")
    return codes, scales, ts, codes_t, scales_t


def dequantize(codes, scales, s_enc):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_dequantize(_ptr(codes), _ptr(scales), float(s_enc), rows, cols, _ptr(out)),
           "dequantize")
    return out


def gemm(a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc):
    """Full C = deq(A) deq(B)^T in double, and sum_k |a_ik b_jk|."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    c = np.empty((M, N), dtype=np.float64)
    cabs = np.empty((M, N), dtype=np.float64)
    _check(lib().orc_gemm(_ptr(a_codes), _ptr(a_scales), float(a_s_enc), _ptr(b_codes),
                          _ptr(b_scales), float(b_s_enc), M, N, K, _ptr(c), _ptr(cabs)), "gemm")
    return c, cabs


def gemm_sample(a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, ii, jj):
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    c = np.empty(len(ii), dtype=np.float64)
    cabs = np.empty(len(ii), dtype=np.float64)
    _check(lib().orc_gemm_sample(_ptr(a_codes), _ptr(a_scales), float(a_s_enc), _ptr(b_codes),
                                 _ptr(b_scales), float(b_s_enc), M, N, K, _ptr(ii), _ptr(jj),
                                 len(ii), _ptr(c), _ptr(cabs)), "gemm_sample")
    return c, cabs


def gemm_dense(a_codes, a_scales, a_s_enc, b_codes, b_scales, b_s_enc, rows=None, chunk=1024):
    """The GEMM definition for every output of a large product: each operand
    is dequantized by the oracle's per-element rule (``dequantize``, the
    value e2m1 * e4m3 / S of every element, in double), and the two are
    contracted in float64 by numpy's matrix product, which also gives
    sum_k |a_ik b_jk| as |A| |B|^T.  Only the order of the double-precision
    additions differs from ``gemm`` (relative difference ~1e-13, far inside
    any fp32 tolerance).  rows (optional) selects the output rows; A is
    processed ``chunk`` rows at a time.  Returns (C, sum |ab|)."""
    a = dequantize(a_codes, a_scales, a_s_enc)
    b = dequantize(b_codes, b_scales, b_s_enc)
    if rows is not None:
        a = a[np.asarray(rows)]
    bt, bat = np.ascontiguousarray(b.T), np.ascontiguousarray(np.abs(b).T)
    del b
    c = np.empty((a.shape[0], bt.shape[1]), dtype=np.float64)
    cabs = np.empty_like(c)
    for r0 in range(0, a.shape[0], chunk):
        blk = a[r0:r0 + chunk]
        np.matmul(blk, bt, out=c[r0:r0 + chunk])
        np.matmul(np.abs(blk), bat, out=cabs[r0:r0 + chunk])
    return c, cabs


def num_threads():
    return lib().orc_num_threads()


# --- MXFP4 ---------------------------------------------------------------
def mx_quantize(x):
    """Returns (codes [rows][cols/2], scales [rows][cols/32] E8M0 bytes)."""
    x, dt = _input(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    _check(lib().orc_mx_quantize(_ptr(x), dt, rows, cols, _ptr(codes), _ptr(scales)), "mx_quantize")
    return codes, scales


def e8m0_value(byte):
    return lib().orc_e8m0_value(int(byte))


def mx_dequantize(codes, scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    out = np.empty((rows, cols), dtype=np.float64)
    _check(lib().orc_mx_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(out)), "mx_dequantize")
    return out


def mx_gemm(a_codes, a_scales, b_codes, b_scales, ii=None, jj=None):
    """C = deq(A) deq(B)^T in double (all of it, or at the (ii, jj) pairs),
    and sum_k |a_ik b_jk| at the same positions."""
    a_codes = np.ascontiguousarray(a_codes, dtype=np.uint8)
    b_codes = np.ascontiguousarray(b_codes, dtype=np.uint8)
    a_scales = np.ascontiguousarray(a_scales, dtype=np.uint8)
    b_scales = np.ascontiguousarray(b_scales, dtype=np.uint8)
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = b_codes.shape[0]
    if ii is None:
        count = M * N
        c = np.empty((M, N), dtype=np.float64)
        a = np.empty((M, N), dtype=np.float64)
        pi = pj = None
    else:
        pi = np.ascontiguousarray(ii, dtype=np.int64)
        pj = np.ascontiguousarray(jj, dtype=np.int64)
        count = pi.size
        c = np.empty(count, dtype=np.float64)
        a = np.empty(count, dtype=np.float64)
    _check(lib().orc_mx_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), M, N, K,
                             _ptr(pi), _ptr(pj), count, _ptr(c), _ptr(a)), "mx_gemm")
    return c, a
