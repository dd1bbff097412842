"""The Python marshallers check every tensor argument (dtype, exact shape or
minimum size, device, layout) before any pointer reaches the library, so an
undersized or mistyped output raises instead of being written past its end.
These run on the CPU: each call below fails its shape or dtype check before
the binding would look for GPU memory, and a call whose arguments are all
well formed fails only on the GPU-memory check."""
import pytest
import torch

import bit_block_scaled_quant_amd as nv

U8, F32, BF16 = torch.uint8, torch.float32, torch.bfloat16


def z(*shape, dtype=U8):
    return torch.zeros(*shape, dtype=dtype)


def well_formed_quantize(rows=32, cols=64, transposed=True):
    x = z(rows, cols, dtype=BF16)
    args = dict(codes=z(rows, cols // 2), scales=z(rows, cols // 16), tensor_scale=z(2, dtype=F32))
    if transposed:
        args.update(codes_t=z(cols, rows // 2), scales_t=z(cols, rows // 16))
    return x, args


def test_well_formed_call_reaches_the_gpu_check():
    x, a = well_formed_quantize()
    with pytest.raises(ValueError, match="GPU memory"):
        nv.nvfp4_quantize(x, 0, 0, 0, 0, **a)


@pytest.mark.parametrize("name,bad", [
    ("codes", z(32, 31)), ("codes", z(31, 32)), ("codes", z(32, 32, dtype=torch.int8)),
    ("scales", z(32, 3)), ("tensor_scale", z(1, dtype=F32)), ("tensor_scale", z(2, dtype=torch.float64)),
    ("codes_t", z(64, 15)), ("scales_t", z(64, 1)), ("scales_t", z(64, 2, dtype=F32)),
])
def test_quantize_rejects_bad_outputs(name, bad):
    x, a = well_formed_quantize()
    a[name] = bad
    with pytest.raises(ValueError, match=name):
        nv.nvfp4_quantize(x, 0, 0, 0, 0, **a)


def test_quantize_rejects_bad_inputs():
    _, a = well_formed_quantize()
    with pytest.raises(ValueError, match="x must be"):
        nv.nvfp4_quantize(z(32, 64, dtype=torch.float16), 0, 0, 0, 0, **a)
    with pytest.raises(ValueError, match="2-D"):
        nv.nvfp4_quantize(z(32 * 64, dtype=F32), 0, 0, 0, 0, **a)
    x, a = well_formed_quantize()
    with pytest.raises(ValueError, match="together"):
        nv.nvfp4_quantize(x, 0, 0, 0, 0, a["codes"], a["scales"], a["tensor_scale"], a["codes_t"], None)
    with pytest.raises(ValueError, match="contiguous"):
        nv.nvfp4_quantize(x, 0, 0, 0, 0, a["codes"], a["scales"], a["tensor_scale"],
                          z(16, 64).t(), a["scales_t"])


def test_quantize_2d_and_cast_transpose():
    x, a = well_formed_quantize()
    a["codes_t"] = z(64, 8)
    with pytest.raises(ValueError, match="codes_t"):
        nv.nvfp4_quantize_2d(x, 0, 0, **a)
    x, a = well_formed_quantize()
    with pytest.raises(ValueError, match="required"):
        nv.nvfp4_quantize_cast_transpose(x, 0, 0, 1, 1, 0, a["codes"], a["scales"], a["tensor_scale"],
                                         None, None, z(2, dtype=F32))
    with pytest.raises(ValueError, match="tensor_scale_t"):
        nv.nvfp4_quantize_cast_transpose(x, 0, 0, 1, 1, 0, a["codes"], a["scales"], a["tensor_scale"],
                                         a["codes_t"], a["scales_t"], z(1, dtype=F32))
    with pytest.raises(ValueError, match="GPU memory"):
        nv.nvfp4_quantize_cast_transpose(x, 0, 0, 1, 1, 0, a["codes"], a["scales"], a["tensor_scale"],
                                         a["codes_t"], a["scales_t"], z(2, dtype=F32))


def test_rht_and_dequantize():
    x = z(16, 32, dtype=F32)
    with pytest.raises(ValueError, match="y must"):
        nv.nvfp4_rht(x, 0, z(16, 16, dtype=F32))
    with pytest.raises(ValueError, match="y must"):
        nv.nvfp4_rht(x, 0, z(16, 32, dtype=BF16))
    codes, scales, ts = z(16, 16), z(16, 2), z(2, dtype=F32)
    with pytest.raises(ValueError, match="out"):
        nv.nvfp4_dequantize(codes, scales, ts, 16, 32, z(16, 31, dtype=F32))
    with pytest.raises(ValueError, match="codes"):
        nv.nvfp4_dequantize(z(16, 8), scales, ts, 16, 32, z(16, 32, dtype=F32))
    with pytest.raises(ValueError, match="GPU memory"):
        nv.nvfp4_dequantize(codes, scales, ts, 16, 32, z(16, 32, dtype=BF16))


def gemm_args(M=32, N=48, K=64, block=16):
    return dict(a_codes=z(M, K // 2), a_scales=z(M, K // block), b_codes=z(N, K // 2),
                b_scales=z(N, K // block))


def test_gemm_rejects_bad_output_and_operands():
    g = gemm_args()
    ts = z(2, dtype=F32)
    call = lambda c, **kw: nv.nvfp4_gemm(kw.get("a_codes", g["a_codes"]), kw.get("a_scales", g["a_scales"]),
                                         ts, kw.get("b_codes", g["b_codes"]), g["b_scales"],
                                         kw.get("b_ts", ts), 32, 48, 64, c)
    with pytest.raises(ValueError, match="c must have shape"):
        call(z(32, 47, dtype=F32))
    with pytest.raises(ValueError, match="c must be"):
        call(z(32, 48, dtype=BF16))  # nvfp4_gemm writes fp32
    with pytest.raises(ValueError, match="a_codes"):
        call(z(32, 48, dtype=F32), a_codes=z(32, 31))
    with pytest.raises(ValueError, match="b_codes"):
        call(z(32, 48, dtype=F32), b_codes=z(47, 32))
    with pytest.raises(ValueError, match="b_tensor_scale"):
        call(z(32, 48, dtype=F32), b_ts=z(0, dtype=F32))
    with pytest.raises(ValueError, match="GPU memory"):
        call(z(32, 48, dtype=F32))


def test_gemm_ex_and_mx():
    g = gemm_args()
    ts = z(2, dtype=F32)
    with pytest.raises(ValueError, match="c_amax"):
        nv.nvfp4_gemm_ex(g["a_codes"], g["a_scales"], ts, g["b_codes"], g["b_scales"], ts, 32, 48, 64,
                         z(32, 48, dtype=BF16), 0.0, z(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU memory"):
        nv.nvfp4_gemm_ex(g["a_codes"], g["a_scales"], ts, g["b_codes"], g["b_scales"], ts, 32, 48, 64,
                         z(32, 48, dtype=BF16), 0.0, z(1, dtype=F32))
    m = gemm_args(block=32)
    with pytest.raises(ValueError, match="a_scales"):
        nv.mxfp4_gemm(m["a_codes"], z(32, 4), m["b_codes"], m["b_scales"], 32, 48, 64, z(32, 48, dtype=F32))
    with pytest.raises(ValueError, match="scales"):
        nv.mxfp4_quantize(z(32, 64, dtype=F32), z(32, 32), z(32, 4))
    with pytest.raises(ValueError, match="out"):
        nv.mxfp4_dequantize(z(32, 32), z(32, 2), 32, 64, z(32, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="GPU memory"):
        nv.mxfp4_quantize(z(32, 64, dtype=F32), z(32, 32), z(32, 2))
