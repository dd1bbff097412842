"""NVFP4 quantizer and block-scaled FP4 GEMM for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libnvfp4.so`` (C ABI in ``include/nvfp4.h``).
The functions named like the C entry points (``nvfp4_quantize``,
``nvfp4_quantize_2d``, ``nvfp4_quantize_cast_transpose``, ``nvfp4_rht``,
``nvfp4_dequantize``, ``nvfp4_gemm``, ``nvfp4_gemm_ex``,
``nvfp4_quantize_with_amax``, and ``mxfp4_quantize``,
``mxfp4_dequantize``, ``mxfp4_gemm``) only marshal torch
tensors into pointers and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing, or a tensor is not on the GPU, the call raises.

Convenience wrappers (``quantize``, ``quantize_2d``,
``quantize_cast_transpose``, ``rht``, ``dequantize``, ``gemm``, ``mx_quantize``,
``mx_dequantize``, ``mx_gemm``)
allocate the outputs with torch (device memory only) and call the same
entry points.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

F32, BF16 = 0, 1
RNE, SR = 0, 1
STATUS = {0: "ok", -1: "invalid argument", -2: "invalid shape", -3: "misaligned pointer",
          -4: "HIP error"}

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status, where, detail=""):
        self.status = status
        msg = f"{where}: {STATUS.get(status, status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


def lib():
    """Load libnvfp4.so (built by ``build.py``); raise if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run bit_block_scaled_quant_amd/build.py "
                              "(hipcc, gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, U64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int
        L.nvfp4_quantize.restype = I
        L.nvfp4_quantize.argtypes = [P, I, I64, I64, I, U64, I, U64, P, P, P, P, P, P]
        L.nvfp4_quantize_2d.restype = I
        L.nvfp4_quantize_2d.argtypes = [P, I, I64, I64, I, U64, P, P, P, P, P, P]
        L.nvfp4_quantize_cast_transpose.restype = I
        L.nvfp4_quantize_cast_transpose.argtypes = [P, I, I64, I64, I, U64, U64, I, U64, P, P, P, P, P, P,
                                                    P]
        L.nvfp4_rht.restype = I
        L.nvfp4_rht.argtypes = [P, I, I64, I64, U64, P, P]
        L.nvfp4_dequantize.restype = I
        L.nvfp4_dequantize.argtypes = [P, P, P, I64, I64, I, P, P]
        L.nvfp4_gemm.restype = I
        L.nvfp4_gemm.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, P]
        L.nvfp4_gemm_ex.restype = I
        L.nvfp4_gemm_ex.argtypes = [P, P, P, P, P, P, I64, I64, I64, P, I, ctypes.c_float, P, P]
        L.nvfp4_quantize_with_amax.restype = I
        L.nvfp4_quantize_with_amax.argtypes = [P, I, I64, I64, I, U64, I, U64, P, P, P, P]
        L.mxfp4_quantize.restype = I
        L.mxfp4_quantize.argtypes = [P, I, I64, I64, P, P, P]
        L.mxfp4_dequantize.restype = I
        L.mxfp4_dequantize.argtypes = [P, P, I64, I64, I, P, P]
        L.mxfp4_gemm.restype = I
        L.mxfp4_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, P]
        L.nvfp4_status_string.restype = ctypes.c_char_p
        L.nvfp4_status_string.argtypes = [I]
        L.nvfp4_last_error.restype = ctypes.c_char_p
        L.nvfp4_last_error.argtypes = []
        _lib = L
    return _lib


def _check(rc, where):
    if rc != 0:
        detail = lib().nvfp4_last_error().decode() if rc == -4 else ""
        raise Nvfp4Error(rc, where, detail)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("nvfp4: tensors must live in GPU memory (no CPU path)")
    if not t.is_contiguous():
        raise ValueError("nvfp4: tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dtype(x: torch.Tensor):
    if x.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16:
        return BF16
    raise TypeError("nvfp4: input must be float32 or bfloat16")


_U8, _F32 = (torch.uint8,), (torch.float32,)
_IN = (torch.float32, torch.bfloat16)


def _want(t, name, dtypes, device, shape=None, min_numel=None, optional=False):
    """Check one tensor argument before any pointer reaches the library: its
    dtype, its exact shape (or at least min_numel elements), its device and
    its layout.  An undersized or mistyped output would otherwise be written
    past its end by a kernel."""
    if t is None:
        if optional:
            return
        raise ValueError(f"nvfp4: {name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"nvfp4: {name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"nvfp4: {name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"nvfp4: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"nvfp4: {name} needs at least {min_numel} elements, got {t.numel()}")
    if t.device != device:
        raise ValueError(f"nvfp4: {name} is on {t.device}, the call's tensors are on {device}")
    if not t.is_contiguous():
        raise ValueError(f"nvfp4: {name} must be contiguous")


def _want_input(x, name="x"):
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError(f"nvfp4: {name} must be a 2-D tensor")
    _want(x, name, _IN, x.device)
    return x.shape[0], x.shape[1], x.device


def _want_quantized(rows, cols, device, codes, scales, tensor_scale, codes_t=None, scales_t=None,
                    block=16, transposed_optional=True):
    _want(codes, "codes", _U8, device, (rows, cols // 2))
    _want(scales, "scales", _U8, device, (rows, cols // block))
    if tensor_scale is not None or block == 16:
        _want(tensor_scale, "tensor_scale", _F32, device, min_numel=2)
    if (codes_t is None) != (scales_t is None):
        raise ValueError("nvfp4: codes_t and scales_t go together (both or neither)")
    if codes_t is None and not transposed_optional:
        raise ValueError("nvfp4: codes_t and scales_t are required")
    _want(codes_t, "codes_t", _U8, device, (cols, rows // 2), optional=True)
    _want(scales_t, "scales_t", _U8, device, (cols, rows // 16), optional=True)


def _want_gemm_operands(a_codes, a_scales, b_codes, b_scales, M, N, K, device, block=16):
    _want(a_codes, "a_codes", _U8, device, (M, K // 2))
    _want(a_scales, "a_scales", _U8, device, (M, K // block))
    _want(b_codes, "b_codes", _U8, device, (N, K // 2))
    _want(b_scales, "b_scales", _U8, device, (N, K // block))


# ---- entry points with the C names (argument marshalling only) ----------
def nvfp4_quantize(x, rounding, seed, rht, rht_seed, codes, scales, tensor_scale,
                   codes_t=None, scales_t=None):
    rows, cols, dev = _want_input(x)
    _want_quantized(rows, cols, dev, codes, scales, tensor_scale, codes_t, scales_t)
    _check(lib().nvfp4_quantize(_ptr(x), _dtype(x), rows, cols, int(rounding), int(seed),
                                int(rht), int(rht_seed), _ptr(codes), _ptr(scales),
                                _ptr(tensor_scale), _ptr(codes_t), _ptr(scales_t), _stream(x)),
           "nvfp4_quantize")


def nvfp4_quantize_2d(w, rounding, seed, codes, scales, tensor_scale, codes_t=None, scales_t=None):
    rows, cols, dev = _want_input(w, "w")
    _want_quantized(rows, cols, dev, codes, scales, tensor_scale, codes_t, scales_t)
    _check(lib().nvfp4_quantize_2d(_ptr(w), _dtype(w), rows, cols, int(rounding), int(seed),
                                   _ptr(codes), _ptr(scales), _ptr(tensor_scale), _ptr(codes_t),
                                   _ptr(scales_t), _stream(w)), "nvfp4_quantize_2d")


def nvfp4_quantize_cast_transpose(x, rounding, seed, seed_t, rht_t, rht_seed, codes, scales, tensor_scale,
                                  codes_t, scales_t, tensor_scale_t):
    rows, cols, dev = _want_input(x)
    _want_quantized(rows, cols, dev, codes, scales, tensor_scale, codes_t, scales_t,
                    transposed_optional=False)
    _want(tensor_scale_t, "tensor_scale_t", _F32, dev, min_numel=2)
    _check(lib().nvfp4_quantize_cast_transpose(
        _ptr(x), _dtype(x), rows, cols, int(rounding), int(seed), int(seed_t), int(rht_t), int(rht_seed),
        _ptr(codes), _ptr(scales), _ptr(tensor_scale), _ptr(codes_t), _ptr(scales_t), _ptr(tensor_scale_t),
        _stream(x)), "nvfp4_quantize_cast_transpose")


def nvfp4_rht(x, rht_seed, y):
    rows, cols, dev = _want_input(x)
    _want(y, "y", _F32, dev, (rows, cols))
    _check(lib().nvfp4_rht(_ptr(x), _dtype(x), rows, cols, int(rht_seed), _ptr(y), _stream(x)),
           "nvfp4_rht")


def nvfp4_dequantize(codes, scales, tensor_scale, rows, cols, out):
    _want(out, "out", _IN, out.device if isinstance(out, torch.Tensor) else None, (rows, cols))
    _want_quantized(rows, cols, out.device, codes, scales, tensor_scale)
    _check(lib().nvfp4_dequantize(_ptr(codes), _ptr(scales), _ptr(tensor_scale), int(rows), int(cols),
                                  _dtype(out), _ptr(out), _stream(out)), "nvfp4_dequantize")


def nvfp4_gemm(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, M, N, K, c):
    _want(c, "c", _F32, c.device if isinstance(c, torch.Tensor) else None, (M, N))
    _want_gemm_operands(a_codes, a_scales, b_codes, b_scales, M, N, K, c.device)
    _want(a_tensor_scale, "a_tensor_scale", _F32, c.device, min_numel=1)
    _want(b_tensor_scale, "b_tensor_scale", _F32, c.device, min_numel=1)
    _check(lib().nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), _ptr(b_codes),
                            _ptr(b_scales), _ptr(b_tensor_scale), int(M), int(N), int(K), _ptr(c),
                            _stream(c)), "nvfp4_gemm")


def nvfp4_gemm_ex(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, M, N, K, c,
                  beta=0.0, c_amax=None):
    _want(c, "c", _IN, c.device if isinstance(c, torch.Tensor) else None, (M, N))
    _want_gemm_operands(a_codes, a_scales, b_codes, b_scales, M, N, K, c.device)
    _want(a_tensor_scale, "a_tensor_scale", _F32, c.device, min_numel=1)
    _want(b_tensor_scale, "b_tensor_scale", _F32, c.device, min_numel=1)
    _want(c_amax, "c_amax", _F32, c.device, min_numel=1, optional=True)
    _check(lib().nvfp4_gemm_ex(_ptr(a_codes), _ptr(a_scales), _ptr(a_tensor_scale), _ptr(b_codes),
                               _ptr(b_scales), _ptr(b_tensor_scale), int(M), int(N), int(K), _ptr(c),
                               _dtype(c), float(beta), _ptr(c_amax), _stream(c)), "nvfp4_gemm_ex")


def nvfp4_quantize_with_amax(x, rounding, seed, rht, rht_seed, codes, scales, tensor_scale):
    rows, cols, dev = _want_input(x)
    _want_quantized(rows, cols, dev, codes, scales, tensor_scale)
    _check(lib().nvfp4_quantize_with_amax(_ptr(x), _dtype(x), rows, cols, int(rounding), int(seed), int(rht),
                                          int(rht_seed), _ptr(codes), _ptr(scales), _ptr(tensor_scale),
                                          _stream(x)), "nvfp4_quantize_with_amax")


def mxfp4_quantize(x, codes, scales):
    rows, cols, dev = _want_input(x)
    _want_quantized(rows, cols, dev, codes, scales, None, block=32)
    _check(lib().mxfp4_quantize(_ptr(x), _dtype(x), rows, cols, _ptr(codes), _ptr(scales), _stream(x)),
           "mxfp4_quantize")


def mxfp4_dequantize(codes, scales, rows, cols, out):
    _want(out, "out", _IN, out.device if isinstance(out, torch.Tensor) else None, (rows, cols))
    _want_quantized(rows, cols, out.device, codes, scales, None, block=32)
    _check(lib().mxfp4_dequantize(_ptr(codes), _ptr(scales), int(rows), int(cols), _dtype(out), _ptr(out),
                                  _stream(out)), "mxfp4_dequantize")


def mxfp4_gemm(a_codes, a_scales, b_codes, b_scales, M, N, K, c):
    _want(c, "c", _F32, c.device if isinstance(c, torch.Tensor) else None, (M, N))
    _want_gemm_operands(a_codes, a_scales, b_codes, b_scales, M, N, K, c.device, block=32)
    _check(lib().mxfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(b_codes), _ptr(b_scales), int(M), int(N),
                            int(K), _ptr(c), _stream(c)), "mxfp4_gemm")


# ---- convenience wrappers ---------------------------------------------------
@dataclass
class Quantized:
    """An NVFP4 tensor of rows x cols quantized along cols (+ optional transpose)."""
    codes: torch.Tensor          # uint8 [rows][cols/2]
    scales: torch.Tensor         # uint8 [rows][cols/16]
    tensor_scale: torch.Tensor   # float32 [2] = (S_enc, amax)
    codes_t: Optional[torch.Tensor] = None   # uint8 [cols][rows/2]
    scales_t: Optional[torch.Tensor] = None  # uint8 [cols][rows/16]

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)

    def transposed(self) -> "Quantized":
        if self.codes_t is None:
            raise ValueError("no transposed copy was produced")
        return Quantized(self.codes_t, self.scales_t, self.tensor_scale)


def _alloc(rows, cols, device, transposed):
    u8 = dict(dtype=torch.uint8, device=device)
    q = Quantized(torch.empty(rows, cols // 2, **u8), torch.empty(rows, cols // 16, **u8),
                  torch.empty(2, dtype=torch.float32, device=device))
    if transposed:
        q.codes_t = torch.empty(cols, rows // 2, **u8)
        q.scales_t = torch.empty(cols, rows // 16, **u8)
    return q


def quantize(x, rounding=RNE, seed=0, rht=False, rht_seed=0, transposed=False) -> Quantized:
    rows, cols = x.shape
    q = _alloc(rows, cols, x.device, transposed)
    nvfp4_quantize(x, rounding, seed, int(rht), rht_seed, q.codes, q.scales, q.tensor_scale,
                   q.codes_t, q.scales_t)
    return q


def quantize_2d(w, rounding=RNE, seed=0, transposed=True) -> Quantized:
    rows, cols = w.shape
    q = _alloc(rows, cols, w.device, transposed)
    nvfp4_quantize_2d(w, rounding, seed, q.codes, q.scales, q.tensor_scale, q.codes_t, q.scales_t)
    return q


def quantize_cast_transpose(x, rounding=RNE, seed=0, seed_t=1, rht_t=True, rht_seed=0):
    """(rowwise, columnwise): the quantization of x [rows][cols] along cols,
    and that of x^T [cols][rows] (with the Hadamard transform when rht_t),
    each with its own tensor scale, from one cast-transpose call."""
    rows, cols = x.shape
    q = _alloc(rows, cols, x.device, False)
    qt = _alloc(cols, rows, x.device, False)
    nvfp4_quantize_cast_transpose(x, rounding, seed, seed_t, int(rht_t), rht_seed, q.codes, q.scales,
                                  q.tensor_scale, qt.codes, qt.scales, qt.tensor_scale)
    return q, qt


def rht(x, rht_seed=0):
    y = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    nvfp4_rht(x, rht_seed, y)
    return y


def dequantize(q: Quantized, dtype=torch.float32):
    """The values q encodes, rows x cols, as float32 or bfloat16."""
    rows, cols = q.shape
    out = torch.empty(rows, cols, dtype=dtype, device=q.codes.device)
    nvfp4_dequantize(q.codes, q.scales, q.tensor_scale, rows, cols, out)
    return out


def gemm(a: Quantized, b: Quantized, out=None):
    """C = deq(a) . deq(b)^T, fp32 [M][N]."""
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError(f"K mismatch: {K} vs {K2}")
    c = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=a.codes.device)
    nvfp4_gemm(a.codes, a.scales, a.tensor_scale, b.codes, b.scales, b.tensor_scale, M, N, K, c)
    return c


@dataclass
class MxQuantized:
    """An MXFP4 tensor of rows x cols quantized along cols."""
    codes: torch.Tensor   # uint8 [rows][cols/2]
    scales: torch.Tensor  # uint8 [rows][cols/32], E8M0

    @property
    def shape(self):
        return (self.codes.shape[0], self.codes.shape[1] * 2)


def mx_quantize(x) -> MxQuantized:
    rows, cols = x.shape
    q = MxQuantized(torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device),
                    torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device))
    mxfp4_quantize(x, q.codes, q.scales)
    return q


def mx_dequantize(q: MxQuantized, dtype=torch.float32):
    rows, cols = q.shape
    out = torch.empty(rows, cols, dtype=dtype, device=q.codes.device)
    mxfp4_dequantize(q.codes, q.scales, rows, cols, out)
    return out


def mx_gemm(a: MxQuantized, b: MxQuantized, out=None):
    """C = deq(a) . deq(b)^T, fp32 [M][N]."""
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError(f"K mismatch: {K} vs {K2}")
    c = out if out is not None else torch.empty(M, N, dtype=torch.float32, device=a.codes.device)
    mxfp4_gemm(a.codes, a.scales, b.codes, b.scales, M, N, K, c)
    return c


def gemm_ex(a: Quantized, b: Quantized, out=None, dtype=torch.float32, beta=0.0, amax=None):
    """C = deq(a) . deq(b)^T + beta * C (fp32 or bf16 C); when amax (a 1-element
    float32 device tensor) is given it receives max |C|."""
    M, K = a.shape
    N, K2 = b.shape
    if K != K2:
        raise ValueError(f"K mismatch: {K} vs {K2}")
    c = out if out is not None else torch.empty(M, N, dtype=dtype, device=a.codes.device)
    nvfp4_gemm_ex(a.codes, a.scales, a.tensor_scale, b.codes, b.scales, b.tensor_scale, M, N, K, c, beta, amax)
    return c
