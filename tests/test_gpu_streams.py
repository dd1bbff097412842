"""Every call enqueues its kernels on the caller's stream and nowhere else.

Two independent layer steps (cast-transposes, the 2D weight quantization
with its transposed copy, three GEMMs) run at the same time on two side
streams.  On each stream the step's inputs are first written by a slow
producer on that same stream, so a kernel launched on any other stream, or
ahead of the producer, would read the stale contents of the input buffers.
Both steps must reproduce, bit for bit, the same steps run one after the
other on the default stream (the quantizers and GEMMs are deterministic).
"""
import pytest
import torch

import bit_block_scaled_quant_amd as nv
from bit_block_scaled_quant_amd import datagen

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
T, H, F = 1024, 1536, 2048  # tokens, hidden, ffn


class Step:
    def __init__(self, seed):
        self.src = [datagen.act(DEV, tokens=T, hidden=H, seed=seed),
                    datagen.weight(DEV, out_features=F, in_features=H, seed=seed + 1),
                    datagen.grad(DEV, tokens=T, out_features=F, seed=seed + 2)]
        self.X, self.W, self.dY = (torch.zeros_like(s) for s in self.src)
        u8 = dict(dtype=torch.uint8, device=DEV)

        def q(rows, cols):
            return nv.Quantized(torch.empty(rows, cols // 2, **u8), torch.empty(rows, cols // 16, **u8),
                                torch.empty(2, dtype=torch.float32, device=DEV))
        self.qX, self.qXt, self.qW, self.qdY, self.qdYt = q(T, H), q(H, T), q(F, H), q(T, F), q(F, T)
        self.qW.codes_t, self.qW.scales_t = torch.empty(H, F // 2, **u8), torch.empty(H, F // 16, **u8)
        self.qWt = nv.Quantized(self.qW.codes_t, self.qW.scales_t, self.qW.tensor_scale)
        self.Y = torch.empty(T, F, dtype=torch.float32, device=DEV)
        self.dX = torch.empty(T, H, dtype=torch.float32, device=DEV)
        self.dW = torch.empty(F, H, dtype=torch.float32, device=DEV)
        self.seed = seed

    def outputs(self):
        return [self.qX.codes, self.qX.scales, self.qX.tensor_scale, self.qXt.codes, self.qXt.scales,
                self.qW.codes, self.qW.codes_t, self.qW.scales, self.qdY.codes, self.qdY.tensor_scale,
                self.qdYt.codes, self.qdYt.scales, self.qdYt.tensor_scale, self.Y, self.dX, self.dW]

    def clear(self):
        for t in (self.X, self.W, self.dY):
            t.zero_()
        for o in self.outputs():
            o.fill_(0x5A if o.dtype == torch.uint8 else -1.0)

    def produce(self, delay):
        """Write the inputs on the current stream, after `delay` passes of
        dummy work on the same stream."""
        junk = torch.empty(32 << 20, dtype=torch.float32, device=DEV)
        for _ in range(delay):
            junk.fill_(1.0)
        for dst, s in zip((self.X, self.W, self.dY), self.src):
            dst.copy_(s)

    def run(self):
        s = self.seed
        nv.nvfp4_quantize_cast_transpose(self.X, 0, 0, 0, 1, s, self.qX.codes, self.qX.scales,
                                         self.qX.tensor_scale, self.qXt.codes, self.qXt.scales,
                                         self.qXt.tensor_scale)
        nv.nvfp4_quantize_2d(self.W, 0, 0, self.qW.codes, self.qW.scales, self.qW.tensor_scale,
                             self.qW.codes_t, self.qW.scales_t)
        nv.gemm(self.qX, self.qW, out=self.Y)
        nv.nvfp4_quantize_cast_transpose(self.dY, 1, s + 1, s + 2, 1, s, self.qdY.codes, self.qdY.scales,
                                         self.qdY.tensor_scale, self.qdYt.codes, self.qdYt.scales,
                                         self.qdYt.tensor_scale)
        nv.gemm(self.qdY, self.qWt, out=self.dX)
        nv.gemm(self.qdYt, self.qXt, out=self.dW)


def test_two_side_streams_match_serial_default_stream():
    steps = [Step(11), Step(23)]
    for st in steps:
        st.produce(0)
        st.run()
    torch.cuda.synchronize()
    want = [[o.clone() for o in st.outputs()] for st in steps]
    for st in steps:
        st.clear()
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for st, s in zip(steps, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            st.produce(40)
            st.run()
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    for k, (st, w) in enumerate(zip(steps, want)):
        for i, (got, ref) in enumerate(zip(st.outputs(), w)):
            assert torch.equal(got, ref), f"step {k}, output {i} differs from the serial run"
