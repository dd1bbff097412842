"""The layer step's calls are safe to capture in a HIP graph: no memsets, no
allocation, no host synchronization, all work on the caller's stream.  A
small fprop + dgrad + wgrad step (cast-transposes, 2D weight quantization
with its transposed copy, three GEMMs) is captured once and replayed three
times, with other eager work and synchronizations between replays, and every
replay must reproduce the eager step's outputs bit for bit (the quantizers
and GEMMs are deterministic)."""
import pytest
import torch

import bit_block_scaled_quant_amd as nv
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
T, H, F = 512, 768, 1024  # tokens, hidden, ffn


def make_step():
    X = datagen.act(DEV, tokens=T, hidden=H, seed=1)
    W = datagen.weight(DEV, out_features=F, in_features=H, seed=2)
    dY = datagen.grad(DEV, tokens=T, out_features=F, seed=3)
    u8 = dict(dtype=torch.uint8, device=DEV)

    def q(rows, cols):
        return nv.Quantized(torch.empty(rows, cols // 2, **u8), torch.empty(rows, cols // 16, **u8),
                            torch.empty(2, dtype=torch.float32, device=DEV))
    qX, qXt, qW, qdY, qdYt = q(T, H), q(H, T), q(F, H), q(T, F), q(F, T)
    qW.codes_t, qW.scales_t = torch.empty(H, F // 2, **u8), torch.empty(H, F // 16, **u8)
    qWt = nv.Quantized(qW.codes_t, qW.scales_t, qW.tensor_scale)
    Y = torch.empty(T, F, dtype=torch.float32, device=DEV)
    dX = torch.empty(T, H, dtype=torch.float32, device=DEV)
    dW = torch.empty(F, H, dtype=torch.float32, device=DEV)

    def step():
        nv.nvfp4_quantize_cast_transpose(X, 0, 0, 0, 1, 7, qX.codes, qX.scales, qX.tensor_scale, qXt.codes,
                                         qXt.scales, qXt.tensor_scale)
        nv.nvfp4_quantize_2d(W, 0, 0, qW.codes, qW.scales, qW.tensor_scale, qW.codes_t, qW.scales_t)
        nv.gemm(qX, qW, out=Y)
        nv.nvfp4_quantize_cast_transpose(dY, 1, 5, 6, 1, 7, qdY.codes, qdY.scales, qdY.tensor_scale, qdYt.codes,
                                         qdYt.scales, qdYt.tensor_scale)
        nv.gemm(qdY, qWt, out=dX)
        nv.gemm(qdYt, qXt, out=dW)
    outs = [qX.codes, qXt.codes, qW.codes, qW.codes_t, qdY.codes, qdYt.codes, qdYt.scales, qdYt.tensor_scale,
            Y, dX, dW]
    return step, outs


def test_layer_step_graph_replays_match_eager():
    step, outs = make_step()
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:  # scribble over the outputs so a replay must rewrite them
            o.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o.view(torch.uint8), w.view(torch.uint8)), f"replay {rep}: output {i} differs"
        step()  # eager work between replays
        torch.cuda.synchronize()
