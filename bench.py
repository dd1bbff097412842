"""Benchmark: one NVFP4 training pass of a 12B-class FFN-up linear layer on one
MI355X, through the C ABI.

A step is the whole hot path over one batch of synthetic input resident in
HBM (shapes of a 12B hybrid Mamba-Transformer layer, "Pretraining Large
Language Models with NVFP4", sections 2B and 3):
  fprop  quantize X [8192x5120] (1D, RNE); quantize W [20480x5120] (2D 16x16,
         RNE, + transposed copy); Y = X . W^T            (M, N, K = 8192, 20480, 5120)
  dgrad  quantize dY [8192x20480] (1D, SR); dX = dY . W  (8192, 5120, 20480)
         using W's transposed copy
  wgrad  quantize dY^T [20480x8192] (1D, SR, RHT) and X^T [5120x8192] (1D, RNE,
         RHT); dW = dY^T . X                              (20480, 5120, 8192)
By default X and X^T come from one cast-transpose call on X, and dY and dY^T
from one on dY (nvfp4_quantize_cast_transpose: bit-identical to the separate
calls, without a transposed bf16 copy of X or dY).  --composed times the
five separate quantize calls instead, on transposes made before the timing.
value = GEMM flops of the step (3 x 2MNK) / wall time of the step, quantizers
included.  Per-call times come from HIP events on the launch stream.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 GEMM TFLOPS + quantize GB/s at 12B-layer shapes (% of roofline)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published
FP4_PEAK_TFLOPS = 10100.0       # dense MXFP4 (context only; not usable exactly for NVFP4)
TOKENS, HIDDEN, FFN = 8192, 5120, 20480


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    # untimed steps first: launches of the same GEMM get faster over the first
    # few tens of milliseconds on the GPU (the clock ramping), and 3 steps
    # left the timed ones about 1.2% slow; 30 (about 130 ms) reach steady state
    p.add_argument("--warmup", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--extras", choices=("all", "none", "only", "sweep"), default="all",
                   help="measurements outside the step (quantizer sweep, dequantize, MXFP4, "
                        "epilogue options, the Tiny workload): all (default), none, only those "
                        "(one untimed step first; prints just the extras), or only the quantizer "
                        "sweep")
    p.add_argument("--graph", action="store_true",
                   help="time the step as replays of one HIP graph instead of eager launches "
                        "(measured +0.2%%: the launches already overlap)")
    p.add_argument("--composed", action="store_true",
                   help="quantize X^T and dY^T by separate calls on materialized transposes "
                        "instead of the cast-transpose")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 256 MiB device copy three times (for scaling the "
                        "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


def quant_bytes(rows, cols, in_bytes, transposed):
    """Algorithmic HBM bytes of one quantize call: the input read twice (amax
    pass, encode pass) plus codes (1/2 B) and scales (1/16 B) per element for
    each copy written."""
    n = rows * cols
    copies = 2 if transposed else 1
    return 2 * in_bytes * n + copies * n * (0.5 + 1.0 / 16.0)


def qmeta(rows, cols, in_bytes, transposed):
    """Bytes of one quantize call: the algorithmic bytes (two reads of the
    input, the method's amax pass then its encode pass) and the single-read
    lower bound (one read of the input), both with every output written."""
    alg = quant_bytes(rows, cols, in_bytes, transposed)
    return {"alg": alg, "one_read": alg - in_bytes * rows * cols}


def gemm_bytes(M, N, K):
    return (M + N) * K * (0.5 + 1.0 / 16.0) + 4.0 * M * N


def traffic_record(kernel_src):
    """HBM bytes per launch measured by rocprofv3 counters, valid only for the
    kernel source they were taken with."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec


def quant_traffic_record():
    """HBM bytes of the step's quantizer calls measured by rocprofv3 counters
    (FETCH_SIZE, WRITE_SIZE, scaled by a plain copy's reading), valid only for
    the sources they were taken with."""
    path = os.path.join(ROOT, "profiles", "quant_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for src in rec.get("sources", []):
        h.update(open(os.path.join(ROOT, src), "rb").read())
    if rec.get("source_sha256") != h.hexdigest():
        return None
    return rec


def cpu_baseline():
    """The oracle, as it stands, on a bounded sample of the same step; its
    per-element / per-output rates are scaled to the full step."""
    import oracle
    from bit_block_scaled_quant_amd import datagen
    t_total = 0.0
    detail = []

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    rows = 1024
    x = datagen.bf16_bits(datagen.act(tokens=rows, hidden=HIDDEN))
    w = datagen.bf16_bits(datagen.weight(out_features=rows, in_features=HIDDEN))
    dy = datagen.bf16_bits(datagen.grad(tokens=rows // 4, out_features=FFN))
    dyt = datagen.bf16_bits(datagen.grad(tokens=rows, out_features=TOKENS))
    xt = datagen.bf16_bits(datagen.act(tokens=rows, hidden=TOKENS))
    quant_jobs = [
        ("X 1D RNE", lambda: oracle.quantize_1d(x), x.size, TOKENS * HIDDEN),
        ("W 2D RNE +T", lambda: oracle.quantize_2d(w), w.size, FFN * HIDDEN),
        ("dY 1D SR", lambda: oracle.quantize_1d(dy, rounding=1), dy.size, TOKENS * FFN),
        ("dYt 1D SR RHT", lambda: oracle.quantize_1d(dyt, rounding=1, rht=1), dyt.size,
         FFN * TOKENS),
        ("Xt 1D RNE RHT", lambda: oracle.quantize_1d(xt, rht=1), xt.size, HIDDEN * TOKENS),
    ]
    for name, fn, n_sample, n_full in quant_jobs:
        dt = timed(fn)
        t_total += dt * n_full / n_sample
        detail.append(f"{name}: {n_sample} of {n_full} elements")
    qx = oracle.quantize_1d(x)
    qw = oracle.quantize_1d(w)
    rng = np.random.default_rng(0)
    for name, (M, N, K) in (("fprop", (TOKENS, FFN, HIDDEN)), ("dgrad", (TOKENS, HIDDEN, FFN)),
                            ("wgrad", (FFN, HIDDEN, TOKENS))):
        # the oracle's cost per output is K multiply-adds; sample at K = 5120
        s = 4096
        ii = rng.integers(0, rows, s)
        jj = rng.integers(0, rows, s)
        dt = timed(lambda: oracle.gemm_sample(qx[0], qx[1], qx[2][0], qw[0], qw[1], qw[2][0], ii, jj))
        per_mac = dt / (s * HIDDEN)
        t_total += per_mac * M * N * K
        detail.append(f"{name}: {s} outputs x {HIDDEN} MACs")
    flops = 3 * 2.0 * TOKENS * FFN * HIDDEN
    # cores: the OpenMP threads the oracle ran with; host_cpus: the logical
    # CPUs of the host and those this process may run on
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "host_cpus": os.cpu_count(),
            "host_cpus_available": len(os.sched_getaffinity(0)),
            "sample": "; ".join(detail) + f"; extrapolated step time {t_total:.1f} s"}


def tiny_times(nv, datagen, torch, dev, reps=50, batch=20):
    """The Tiny workload (A, B [256 x 256] fp32, 1% x50 outliers, seed 0, both
    quantized 1D with RNE, then C = A . B^T): device time per call and per
    pass.  Each call (and the pass) is captured `batch` times back to back in
    one HIP graph; a replay is timed by HIP events on the replay stream and
    divided by `batch`, median of `reps` replays.  Timing single eager calls
    would measure the host's launch latency instead: the GPU idles between
    them.  Latency-bound (one or two waves of work), so no roofline claim."""
    a = datagen.tiny(dev, seed=0, tag=datagen.TAG_A)
    b = datagen.tiny(dev, seed=0, tag=datagen.TAG_B)
    qa, qb = nv.quantize(a), nv.quantize(b)
    c = torch.empty(256, 256, dtype=torch.float32, device=dev)
    calls = {"quantize_A": lambda: nv.nvfp4_quantize(a, 0, 0, 0, 0, qa.codes, qa.scales, qa.tensor_scale),
             "quantize_B": lambda: nv.nvfp4_quantize(b, 0, 0, 0, 0, qb.codes, qb.scales, qb.tensor_scale),
             "gemm": lambda: nv.gemm(qa, qb, out=c)}

    def timed_graph(fns):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for fn in fns:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(batch):
                for fn in fns:
                    fn()
        graph.replay()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / batch)
        return round(float(np.median(ts)), 2)

    out = {name + "_us": timed_graph([fn]) for name, fn in calls.items()}
    out["pass_us"] = timed_graph(list(calls.values()))
    out["shape"] = "A, B [256 x 256] fp32; C = A . B^T 256 x 256 x 256"
    out["timing"] = f"HIP graph of {batch} back-to-back calls, median of {reps} replays, per call"
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the quantizer and GEMM "
              "path is measured on one GPU's share of the layer; nothing here uses a second GPU",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        a = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda:0").fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 4, "repeats": 3}), flush=True)
        return

    import bit_block_scaled_quant_amd as nv
    from bit_block_scaled_quant_amd import build as nvbuild
    from bit_block_scaled_quant_amd import datagen
    if not os.path.exists(nv.LIB_PATH):
        nvbuild.build()
    nv.lib()

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    seed = args.seed
    # dY^T's stochastic rounding draws from a key of its own, so the two SR
    # copies of dY (dgrad's and wgrad's) use independent random bits
    seed_t = seed + 1
    X = datagen.act(dev, seed=seed)
    W = datagen.weight(dev, seed=seed)
    dY = datagen.grad(dev, seed=seed)
    if args.composed:
        dYt = dY.t().contiguous()
        Xt = X.t().contiguous()
    torch.cuda.synchronize()

    def alloc(rows, cols, transposed):
        u8 = dict(dtype=torch.uint8, device=dev)
        q = nv.Quantized(torch.empty(rows, cols // 2, **u8), torch.empty(rows, cols // 16, **u8),
                         torch.empty(2, dtype=torch.float32, device=dev))
        if transposed:
            q.codes_t = torch.empty(cols, rows // 2, **u8)
            q.scales_t = torch.empty(cols, rows // 16, **u8)
        return q

    qX = alloc(TOKENS, HIDDEN, False)
    qW = alloc(FFN, HIDDEN, True)
    qdY = alloc(TOKENS, FFN, False)
    qdYt = alloc(FFN, TOKENS, False)
    qXt = alloc(HIDDEN, TOKENS, False)
    Y = torch.empty(TOKENS, FFN, dtype=torch.float32, device=dev)
    dX = torch.empty(TOKENS, HIDDEN, dtype=torch.float32, device=dev)
    dW = torch.empty(FFN, HIDDEN, dtype=torch.float32, device=dev)
    qWt = nv.Quantized(qW.codes_t, qW.scales_t, qW.tensor_scale)

    quant_W = ("quant_W_2d_rne_t", "quant", lambda: nv.nvfp4_quantize_2d(
        W, 0, 0, qW.codes, qW.scales, qW.tensor_scale, qW.codes_t, qW.scales_t),
        qmeta(FFN, HIDDEN, 2, True))
    gemm_fprop = ("gemm_fprop", "gemm", lambda: nv.gemm(qX, qW, out=Y), (TOKENS, FFN, HIDDEN))
    gemm_dgrad = ("gemm_dgrad", "gemm", lambda: nv.gemm(qdY, qWt, out=dX), (TOKENS, HIDDEN, FFN))
    gemm_wgrad = ("gemm_wgrad", "gemm", lambda: nv.gemm(qdYt, qXt, out=dW), (FFN, HIDDEN, TOKENS))
    if args.composed:
        calls = [
            ("quant_X_1d_rne", "quant", lambda: nv.nvfp4_quantize(X, 0, 0, 0, 0, qX.codes, qX.scales,
                                                                  qX.tensor_scale),
             qmeta(TOKENS, HIDDEN, 2, False)),
            quant_W, gemm_fprop,
            ("quant_dY_1d_sr", "quant", lambda: nv.nvfp4_quantize(dY, 1, seed, 0, 0, qdY.codes,
                                                                  qdY.scales, qdY.tensor_scale),
             qmeta(TOKENS, FFN, 2, False)),
            gemm_dgrad,
            ("quant_dYt_1d_sr_rht", "quant", lambda: nv.nvfp4_quantize(
                dYt, 1, seed_t, 1, seed, qdYt.codes, qdYt.scales, qdYt.tensor_scale),
             qmeta(FFN, TOKENS, 2, False)),
            ("quant_Xt_1d_rne_rht", "quant", lambda: nv.nvfp4_quantize(
                Xt, 0, 0, 1, seed, qXt.codes, qXt.scales, qXt.tensor_scale),
             qmeta(HIDDEN, TOKENS, 2, False)),
            gemm_wgrad,
        ]
    else:
        # the same outputs as the composed calls (same seeds), bit for bit
        calls = [
            ("ct_X_rne_rht", "quant", lambda: nv.nvfp4_quantize_cast_transpose(
                X, 0, 0, 0, 1, seed, qX.codes, qX.scales, qX.tensor_scale, qXt.codes, qXt.scales,
                qXt.tensor_scale), qmeta(TOKENS, HIDDEN, 2, True)),
            quant_W, gemm_fprop,
            ("ct_dY_sr_rht", "quant", lambda: nv.nvfp4_quantize_cast_transpose(
                dY, 1, seed, seed_t, 1, seed, qdY.codes, qdY.scales, qdY.tensor_scale, qdYt.codes,
                qdYt.scales, qdYt.tensor_scale), qmeta(TOKENS, FFN, 2, True)),
            gemm_dgrad, gemm_wgrad,
        ]

    def step(events=None):
        for i, (_, _, fn, _) in enumerate(calls):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    def run_sweep(reps=5):
        """The quantizer-only bandwidth sweep: bf16 N(0,1) with 0.1% of the
        entries x100 at three shapes, each quantized 1D with its columnwise
        copy and 2D with its transposed copy, with RNE and with SR.  Every
        timed call starts from a cold cache: a 512 MiB write and then a read
        of those 512 MiB evict the input from L2 and the 256 MB MALL first.
        The read leaves the caches holding clean lines only: after the write
        alone, the timed call would also pay for writing the flush's dirty
        lines back to HBM (measured: 10-30 us on the large calls).  The time
        is the median of the calls (HIP events on the launch stream around
        the call alone)."""
        flush = torch.empty(128 * 1024 * 1024, dtype=torch.float32, device=dev)
        res = {}
        for rows, cols in ((TOKENS, HIDDEN), (TOKENS, FFN), (4 * TOKENS, HIDDEN)):
            xs = datagen.sweep(rows, cols, device=dev, seed=seed)
            qs = alloc(rows, cols, True)
            for two_d in (False, True):
                for rnd in (0, 1):
                    if two_d:
                        fn = lambda: nv.nvfp4_quantize_2d(xs, rnd, seed, qs.codes, qs.scales,
                                                          qs.tensor_scale, qs.codes_t, qs.scales_t)
                    else:
                        fn = lambda: nv.nvfp4_quantize(xs, rnd, seed, 0, 0, qs.codes, qs.scales,
                                                       qs.tensor_scale, qs.codes_t, qs.scales_t)
                    fn()
                    ts = []
                    for _ in range(reps):
                        flush.fill_(float(len(ts)))
                        flush_sum = flush.sum()  # reads the 512 MiB back: evicts the dirty lines
                        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        a.record()
                        fn()
                        b.record()
                        torch.cuda.synchronize()
                        ts.append(a.elapsed_time(b))
                    del flush_sum
                    ms = float(np.median(ts))
                    qm = qmeta(rows, cols, 2, True)
                    gbs = qm["alg"] / (ms * 1e-3) / 1e9
                    key = f"{rows}x{cols}_{'2d' if two_d else '1d'}+t_{'sr' if rnd else 'rne'}"
                    res[key] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                                "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                "frac_hbm_peak_one_read_bound": round(
                                    qm["one_read"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del xs, qs
        del flush
        return res

    def copy_bandwidth(reps=10):
        """A plain 1 GiB device-to-device copy (torch's copy kernel): the HBM
        rate a streaming kernel reaches on this machine, beside the 8 TB/s
        datasheet peak the fractions use.  Bytes = read + write."""
        src = torch.empty(256 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        gbs = 2 * src.numel() * 4 / (ms * 1e-3) / 1e9
        del src, dst
        return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}

    def run_extras():
        """Measurements outside the step (not part of value)."""
        extras = {"copy_1GiB": copy_bandwidth(), "quantizer_sweep": run_sweep(),
                  "tiny": tiny_times(nv, datagen, torch, dev)}
        # outside the step: dequantization of dY's rowwise copy (HBM-bound)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        gemm_flops_one = 2.0 * TOKENS * FFN * HIDDEN

        # GEMM-sized calls get 20 untimed calls first: after the short
        # memory-bound kernels before them the clock ramps up again
        def timed_ms_ev(fn, reps=10, warm=1):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(reps):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / reps
        for dt, out_bytes, tag in ((torch.bfloat16, 2, "bf16"), (torch.float32, 4, "f32")):
            out_t = torch.empty(TOKENS, FFN, dtype=dt, device=dev)

            def deq():
                nv.nvfp4_dequantize(qdY.codes, qdY.scales, qdY.tensor_scale, TOKENS, FFN, out_t)
            deq()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(10):
                deq()
            ev1.record()
            torch.cuda.synchronize()
            ms = ev0.elapsed_time(ev1) / 10
            gbs = TOKENS * FFN * (0.5 + 1.0 / 16.0 + out_bytes) / (ms * 1e-3) / 1e9
            extras[f"dequantize_dY_{tag}"] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                                              "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
            del out_t

        # epilogue options: fprop with bf16 output and the output amax, then the
        # single-read quantization of that output (its amax already known)
        Y16 = torch.empty(TOKENS, FFN, dtype=torch.bfloat16, device=dev)
        tsY = torch.zeros(2, dtype=torch.float32, device=dev)
        ms = timed_ms_ev(lambda: nv.gemm_ex(qX, qW, out=Y16, amax=tsY[1:]), warm=20)
        tf = gemm_flops_one / (ms * 1e-3) / 1e12
        extras["gemm_ex_fprop_bf16_out_amax"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                                                 "frac_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}

        # beta-accumulation (gradient accumulation into an fp32 C): C += A B
        Y32 = torch.zeros(TOKENS, FFN, dtype=torch.float32, device=dev)
        ms = timed_ms_ev(lambda: nv.gemm_ex(qX, qW, out=Y32, beta=1.0), warm=20)
        tf = gemm_flops_one / (ms * 1e-3) / 1e12
        extras["gemm_ex_fprop_f32_beta1"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                                             "frac_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}
        del Y32
        qY = nv.Quantized(torch.empty(TOKENS, FFN // 2, dtype=torch.uint8, device=dev),
                          torch.empty(TOKENS, FFN // 16, dtype=torch.uint8, device=dev), tsY)
        ms = timed_ms_ev(lambda: nv.nvfp4_quantize_with_amax(Y16, 0, 0, 0, 0, qY.codes, qY.scales, tsY))
        gbs = TOKENS * FFN * (2 + 0.5 + 1.0 / 16.0) / (ms * 1e-3) / 1e9
        extras["quantize_with_amax_Y_bf16"] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                                               "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del Y16, qY

        # MXFP4, the format the pages measure NVFP4 against: the same three GEMMs
        # on gfx950's scaled FP4 MFMA, its quantizer, and the quantization error
        # of both formats on the layer's tensors (a dataset-free proxy for the
        # pages' accuracy comparison).  Outside the step.
        def timed_ms(fn, reps=10, warm=1):
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            ev0.record()
            for _ in range(reps):
                fn()
            ev1.record()
            torch.cuda.synchronize()
            return ev0.elapsed_time(ev1) / reps

        Wt = W.t().contiguous()
        dYt_m = dY.t().contiguous()
        Xt_m = X.t().contiguous()
        mx_ops = {"fprop": (X, W), "dgrad": (dY, Wt), "wgrad": (dYt_m, Xt_m)}
        mxq = {}
        for name, (a, b) in mx_ops.items():
            qa, qb = nv.mx_quantize(a), nv.mx_quantize(b)
            M, K = a.shape
            N = b.shape[0]
            cbuf = {"fprop": Y, "dgrad": dX, "wgrad": dW}[name]
            ms = timed_ms(lambda: nv.mx_gemm(qa, qb, out=cbuf), warm=20)
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            extras[f"mxfp4_gemm_{name}"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                                            "frac_fp4_mfma_peak": round(tf / FP4_PEAK_TFLOPS, 4)}
            mxq[name] = (qa, M, K)
        qa, M, K = mxq["dgrad"]
        ms = timed_ms(lambda: nv.mxfp4_quantize(dY, qa.codes, qa.scales))
        gbs = M * K * (2 + 0.5 + 1.0 / 32.0) / (ms * 1e-3) / 1e9
        extras["mxfp4_quantize_dY"] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                                       "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        del Wt, dYt_m, Xt_m, mxq, qa

        def rel_err(t, deq):
            d = (deq.double() - t.double())
            return float(torch.linalg.vector_norm(d) / torch.linalg.vector_norm(t.double()))

        err = {}
        for name, t, two_d in (("X", X, False), ("W", W, True), ("dY", dY, False)):
            qn = nv.quantize_2d(t, transposed=False) if two_d else nv.quantize(t)
            e_nv = rel_err(t, nv.dequantize(qn))
            del qn
            e_mx = rel_err(t, nv.mx_dequantize(nv.mx_quantize(t)))
            err[name] = {"nvfp4": round(e_nv, 5), "mxfp4": round(e_mx, 5)}
        extras["relative_rms_quantization_error"] = err
        return extras

    if args.extras == "sweep":
        print(json.dumps({"extras": {"copy_1GiB": copy_bandwidth(), "quantizer_sweep": run_sweep()}}),
              flush=True)
        return
    if args.extras == "only":
        step()
        torch.cuda.synchronize()
        print(json.dumps({"extras": run_extras()}), flush=True)
        return

    # The step's calls are capture-safe (no memsets, allocation or host
    # synchronization); with --graph the whole step is captured once as a HIP
    # graph and the timed steps are replays of it (the same kernels, without
    # per-launch gaps); tests/test_gpu_graph.py checks that replays reproduce
    # the eager step bit for bit.
    run, graph_note = step, "eager launches"
    if args.graph:
        try:
            warm = torch.cuda.Stream()
            warm.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(warm):
                step()
            torch.cuda.current_stream().wait_stream(warm)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            run, graph_note = graph.replay, "HIP graph replay"
        except Exception as e:  # keep the eager timing
            graph_note = f"eager launches (graph capture failed: {e})"

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # timed steps (no events inside) for the step time
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-call durations with HIP events on the launch stream, recorded over
    # K steps launched back to back and read after one synchronization: each
    # call's start event then completes when the previous call does, so host
    # launch latency (an idle GPU waiting for the next launch) is not counted
    per_call = {name: [] for name, _, _, _ in calls}
    step_events = []
    for _ in range(args.steps):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in calls]
        step(ev)
        step_events.append(ev)
    torch.cuda.synchronize()
    for ev in step_events:
        for (name, _, _, _), (a, b) in zip(calls, ev):
            per_call[name].append(a.elapsed_time(b))

    extras = run_extras() if args.extras == "all" else {}

    gemm_flops = 2.0 * TOKENS * FFN * HIDDEN
    step_flops = 3 * gemm_flops
    components = {}
    gemm_ms = []
    quant_ms_total, quant_bytes_total = 0.0, 0.0
    qrec = quant_traffic_record()
    quant_counter_bytes = 0.0 if qrec else None
    for name, kind, _, meta in calls:
        ms = float(np.median(per_call[name]))
        if kind == "gemm":
            M, N, K = meta
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            gemm_ms.append(ms)
            components[name] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                                "frac_fp16_mfma_peak": round(tf / FP16_MFMA_PEAK_TFLOPS, 4)}
        else:
            gbs = meta["alg"] / (ms * 1e-3) / 1e9
            quant_ms_total += ms
            quant_bytes_total += meta["alg"]
            # frac_hbm_peak_one_read_bound: the same time against the bytes of a
            # single read of the input (what a known amax would allow)
            components[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                                "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                "frac_hbm_peak_one_read_bound": round(
                                    meta["one_read"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            # the HBM bytes the counters saw for this call (profiles/quant_traffic.json)
            c = qrec["calls"].get(name) if qrec else None
            if c is not None:
                cb = c["read_bytes"] + c["write_bytes"]
                quant_counter_bytes += cb
                components[name]["counter_bytes"] = cb
                components[name]["frac_hbm_peak_counters"] = round(cb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            elif qrec is not None:
                quant_counter_bytes = None
                qrec = None

    avg_gemm_ms = float(np.mean(gemm_ms))
    achieved = gemm_flops / (avg_gemm_ms * 1e-3) / 1e12
    rec = traffic_record(os.path.join(ROOT, "bit_block_scaled_quant_amd", "csrc", "gemm.hip"))
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / FP16_MFMA_PEAK_TFLOPS, 4),
                "traffic": (rec["bytes_per_launch"] if rec else None),
                "kernel": "k_gemm_m32<4> (+ k_gemm_m32<2> or <1> for a partial last wave of tiles; fp16 MFMA 32x32x16, fp32 accumulate)",
                "algorithmic_flops_per_launch": gemm_flops,
                "context_frac_of_fp4_peak": round(achieved / FP4_PEAK_TFLOPS, 4)}

    out = {
        "metric": METRIC,
        "value": round(step_flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 operands, fp16 MFMA, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "12B FFN-up linear layer, NVFP4 fprop+dgrad+wgrad",
                   "quantizer_calls": "separate (transposes made before timing)" if args.composed
                   else "cast-transpose for X and dY",
                   "step_launch": graph_note,
                   "X": [TOKENS, HIDDEN], "W": [FFN, HIDDEN], "dY": [TOKENS, FFN],
                   "gemm_MNK": [[TOKENS, FFN, HIDDEN], [TOKENS, HIDDEN, FFN],
                                [FFN, HIDDEN, TOKENS]]},
        "gemm_TFLOPs": round(achieved, 1),
        "quantize_GBps": round(quant_bytes_total / (quant_ms_total * 1e-3) / 1e9, 1),
        "quantize_frac_hbm_peak": round(quant_bytes_total / (quant_ms_total * 1e-3) / 1e9
                                        / HBM_PEAK_GBS, 4),
        # the same time against the HBM bytes the counters measured for these
        # calls (null when the quantizer sources changed since they were taken)
        "quantize_frac_hbm_peak_counters": (round(quant_counter_bytes / (quant_ms_total * 1e-3) / 1e9
                                                  / HBM_PEAK_GBS, 4)
                                            if quant_counter_bytes is not None else None),
        "components": components,
        "extras": extras,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
