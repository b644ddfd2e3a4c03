"""Benchmark: one FP8 blockwise linear training step (fwd + dgrad + wgrad,
quantization included) at M=16640, N=5120, K=8192 on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 200] [--no-cpu-baseline]

The default warm-up (200 steps, about 0.45 s) lets the shader clock settle
at its loaded level: after only 5 warm-up steps the timed steps measured
about 1.5% slower.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM, X and dY each quantized once into both code layouts
(the sequence fp8_linear_fwd_save and fp8_linear_bwd enqueue, which
Float8BlockwiseLinear trains through):
  fwd    quant X -> X (1x128) and X^T (1x128 along M); quant W -> W
         (128x128); GEMM (1x128 x 128x128)                        -> Y  [M, N]
  bwd    quant dY -> dY (1x128) and dY^T (1x128 along M);
         quant W -> W^T (128x128); dgrad GEMM (dY x W^T)          -> dX [M, K]
         wgrad GEMM (dY^T x X^T, 1x128 x 1x128)                    -> dW [N, K]
each call through the C ABI on torch's current stream.  HIP events around
every launch give each kernel's average duration over the timed steps.

Prints one JSON line: `value` is the step's effective throughput,
3 * 2MNK flops / step time (TFLOP/s); `roofline` is for the dominant kernel,
the GEMM call with the largest share of the step's time (2MNK flops per call
/ its average duration between HIP events on the launch stream, vs the 5.0
PFLOP/s dense FP8 peak; a call is its main launch plus, where the plan has
one, the split of the leftover tiles and their reduce); `rooflines` gives the
same for every GEMM call of the step; `cpu_baseline` times the CPU oracle on
a bounded sample of the same workload.  Also reported:
  separate_quant_step   the same step with the six separate quantizer
                        launches of fp8_linear_fwd / _dgrad / _wgrad (X and
                        dY each read twice);
  step_16640x8192x5120  the fused step at the second linear shape (N and K
                        swapped);
  grouped_gemm          the mixture-of-experts grouped GEMM at the forward
                        shape;
  quant_standalone      the quantizers alone on S x S inputs, S = 1024 ..
                        32768 (headline entries at 32768^2);
  tiny_linear           the 128 x 256 x 512 linear step (latency-bound);
  per_tensor            per-tensor quantization of X [256, 1024] and
                        W [4096, 1024] and the tensorwise GEMM, plus the
                        16 x 32 x 32 fp32-out edge case;
  tensorwise_quant      the per-tensor quantizer on large inputs (two passes:
                        5 B moved per element, 3 B algorithmic);
  long_k                the blockwise GEMM at M = N = 1024,
                        K = 128000 / 128128 / 128256 (K split over the chip,
                        then an ordered reduce).
"""

import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blockwise FP8 GEMM TFLOP/s (M16640 N5120 K8192) + quant GB/s, 1 MI355X"
FP8_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (no sparsity)
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
M, N, K = 16640, 5120, 8192
SHAPE2 = (16640, 8192, 5120)


def cdiv(a, b):
    return (a + b - 1) // b


class Workload:
    """Inputs, codes, scales and outputs of one linear step, all in HBM
    (X [M, K], W [N, K], dY [M, N])."""

    def __init__(self, seed, dev, shape=(M, N, K)):
        from synth import inputs
        M, N, K = self.M, self.N, self.K = shape
        self.x = inputs.randn_bf16((M, K), seed=inputs.tensor_seed(seed, "x"), device=dev)
        self.w = inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(seed, "w"), device=dev)
        self.dy = inputs.randn_bf16((M, N), seed=inputs.tensor_seed(seed, "dy"), device=dev)
        u8, f32 = torch.uint8, torch.float32
        e = lambda *s, dt=u8: torch.empty(s, dtype=dt, device=dev)  # noqa: E731
        cm = lambda ni, nj: torch.empty((nj, ni), dtype=f32, device=dev).t()  # noqa: E731
        self.xq, self.xr = e(M, K), cm(M, cdiv(K, 128))
        self.wq, self.wr = e(N, K), cm(cdiv(N, 128), cdiv(K, 128))
        self.dyq, self.dyr = e(M, N), cm(M, cdiv(N, 128))
        self.wtq, self.wtr = e(K, N), cm(cdiv(K, 128), cdiv(N, 128))
        self.dytq, self.dytr = e(N, M), cm(N, cdiv(M, 128))
        self.xtq, self.xtr = e(K, M), cm(K, cdiv(M, 128))
        self.y = e(M, N, dt=torch.bfloat16)
        self.dx = e(M, K, dt=torch.bfloat16)
        self.dw = e(N, K, dt=torch.bfloat16)


def quant_bytes(rows, cols, block):
    nscales = rows * cdiv(cols, 128) if block == "1x128" else cdiv(rows, 128) * cdiv(cols, 128)
    return 2 * rows * cols + rows * cols + 4 * nscales


def step_plan(wl):
    """(kernel label, launch callable, work, unit) for the step with separate
    quantizer launches (fp8_linear_fwd / _dgrad / _wgrad), in order."""
    import blockwise_scaled_fp8_amd as fp8
    q = fp8.fp8_blockwise_quant
    g = fp8.fp8_scaled_gemm_blockwise
    M, N, K = wl.M, wl.N, wl.K
    return [
        ("quant_1x128 X", lambda: q(wl.x, "1x128", q=wl.xq, recip=wl.xr),
         quant_bytes(M, K, "1x128"), "B"),
        ("quant_128x128 W", lambda: q(wl.w, "128x128", q=wl.wq, recip=wl.wr),
         quant_bytes(N, K, "128x128"), "B"),
        ("gemm fwd", lambda: g(wl.xq, wl.xr, wl.wq, wl.wr, "128x128", out=wl.y),
         2 * M * N * K, "flop"),
        ("quant_1x128 dY", lambda: q(wl.dy, "1x128", q=wl.dyq, recip=wl.dyr),
         quant_bytes(M, N, "1x128"), "B"),
        ("quant_128x128^T W", lambda: q(wl.w, "128x128", transpose=True, q=wl.wtq, recip=wl.wtr),
         quant_bytes(N, K, "128x128"), "B"),
        ("gemm dgrad", lambda: g(wl.dyq, wl.dyr, wl.wtq, wl.wtr, "128x128", out=wl.dx),
         2 * M * N * K, "flop"),
        ("quant_1x128^T dY", lambda: q(wl.dy, "1x128", transpose=True, q=wl.dytq, recip=wl.dytr),
         quant_bytes(M, N, "1x128"), "B"),
        ("quant_1x128^T X", lambda: q(wl.x, "1x128", transpose=True, q=wl.xtq, recip=wl.xtr),
         quant_bytes(M, K, "1x128"), "B"),
        ("gemm wgrad", lambda: g(wl.dytq, wl.dytr, wl.xtq, wl.xtr, "1x128", out=wl.dw),
         2 * M * N * K, "flop"),
    ]


def step_plan_dual(wl):
    """The step as fp8_linear_fwd_save / fp8_linear_bwd enqueue it: X -> X
    and X^T codes and dY -> dY and dY^T codes from one read each
    (fp8_blockwise_quant_dual, bit-identical to the separate quantizers; X^T,
    kept for the backward, with nontemporal stores), W -> W codes for the
    forward and W -> W^T codes right before the dgrad GEMM, and the three
    GEMMs."""
    import blockwise_scaled_fp8_amd as fp8
    d = fp8.fp8_blockwise_quant_dual
    q = fp8.fp8_blockwise_quant
    g = fp8.fp8_scaled_gemm_blockwise
    M, N, K = wl.M, wl.N, wl.K
    return [
        ("quant_dual X", lambda: d(wl.x, "1x128", q=wl.xq, recip=wl.xr, qt=wl.xtq, recip_t=wl.xtr,
                                   stream_t=True),
         2 * M * K + 2 * M * K + 4 * (M * cdiv(K, 128) + K * cdiv(M, 128)), "B"),
        ("quant_128x128 W", lambda: q(wl.w, "128x128", q=wl.wq, recip=wl.wr),
         quant_bytes(N, K, "128x128"), "B"),
        ("gemm fwd", lambda: g(wl.xq, wl.xr, wl.wq, wl.wr, "128x128", out=wl.y),
         2 * M * N * K, "flop"),
        ("quant_dual dY", lambda: d(wl.dy, "1x128", q=wl.dyq, recip=wl.dyr, qt=wl.dytq, recip_t=wl.dytr),
         2 * M * N + 2 * M * N + 4 * (M * cdiv(N, 128) + N * cdiv(M, 128)), "B"),
        ("quant_128x128^T W", lambda: q(wl.w, "128x128", transpose=True, q=wl.wtq, recip=wl.wtr),
         quant_bytes(N, K, "128x128"), "B"),
        ("gemm dgrad", lambda: g(wl.dyq, wl.dyr, wl.wtq, wl.wtr, "128x128", out=wl.dx),
         2 * M * N * K, "flop"),
        ("gemm wgrad", lambda: g(wl.dytq, wl.dytr, wl.xtq, wl.xtr, "1x128", out=wl.dw),
         2 * M * N * K, "flop"),
    ]


def run_gpu(steps, warmup, seed, plan_fn=None, wl=None, shape=(M, N, K)):
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    import blockwise_scaled_fp8_amd as fp8
    fp8.load_library()
    if wl is None:
        wl = Workload(seed, dev, shape)
    plan = (plan_fn or step_plan)(wl)
    torch.cuda.synchronize()
    for _ in range(warmup):
        for _, fn, _, _ in plan:
            fn()
    torch.cuda.synchronize()
    n = len(plan)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for s in range(steps):
        evs[s][0].record()
        for i, (_, fn, _, _) in enumerate(plan):
            fn()
            evs[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [0.0] * n
    for s in range(steps):
        for i in range(n):
            per[i] += evs[s][i].elapsed_time(evs[s][i + 1])
    per = [p / steps for p in per]            # ms per launch
    gpu_ms_events = sum(evs[s][0].elapsed_time(evs[s][n]) for s in range(steps)) / steps
    # The same steps again with events only around the whole run: each event
    # recorded between two calls leaves the GPU idle for a few microseconds,
    # so the step time (the headline) comes from this pass and the per-call
    # pass above gives each call's share.
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for s in range(steps):
        for _, fn, _, _ in plan:
            fn()
    e1.record()
    torch.cuda.synchronize()
    gpu_ms = e0.elapsed_time(e1) / steps
    kernels = {}
    for (name, _, work, unit), ms in zip(plan, per):
        rate = work / (ms * 1e-3)
        kernels[name] = ({"avg_us": round(ms * 1e3, 2), "tflops": round(rate / 1e12, 1)}
                         if unit == "flop" else
                         {"avg_us": round(ms * 1e3, 2), "gbps": round(rate / 1e9, 1)})
    qbytes = sum(w for _, _, w, u in plan if u == "B")
    qms = sum(ms for (_, _, _, u), ms in zip(plan, per) if u == "B")
    return {"wall_ms_per_step": wall / steps * 1e3, "gpu_ms_per_step": gpu_ms,
            "gpu_ms_per_step_with_call_events": gpu_ms_events, "per_ms": per,
            "plan": [(nm, w, u) for nm, _, w, u in plan], "kernels": kernels,
            "quant_gbps": qbytes / (qms * 1e-3) / 1e9, "quant_us": qms * 1e3, "workload": wl}


def _time_quant(xs, qs, recips, block, reps, graph=False):
    """Average duration (ms) of one quantizer call, cycling through the
    buffers so consecutive calls touch different memory; one HIP event pair
    around the whole sequence on the launch stream.  With `graph` the
    sequence is captured once as a HIP graph and replayed, so the host's
    per-call cost (Python, argument checks) drops out of the figure."""
    import blockwise_scaled_fp8_amd as fp8
    n = len(xs)
    # Warm-up of at least ~100 ms of calls: right after a single warm-up call
    # a 32768^2 quantizer measured 8% slower than once the clock has settled.
    t0 = time.perf_counter()
    i = 0
    while i < max(3, n) or time.perf_counter() - t0 < 0.1:
        fp8.fp8_blockwise_quant(xs[i % n], block, q=qs[i % n], recip=recips[i % n])
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    calls = max(reps, 2 * n)

    def seq():
        for i in range(calls):
            fp8.fp8_blockwise_quant(xs[i % n], block, q=qs[i % n], recip=recips[i % n])

    g = None
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            seq()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            seq()
        g.replay()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    if g is not None:
        g.replay()
    else:
        seq()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / calls


def quant_standalone(seed, sizes=(1024, 2048, 4096, 8192, 16384, 32768), reps=20,
                     rotate_bytes=1 << 30):
    """The quantizers alone on square S x S bf16 inputs, both block shapes.
    Each size cycles through enough input / output buffer sets that their
    inputs total at least 1 GiB, four times the 256 MB Infinity Cache, so
    every call streams from HBM (32768^2 is one 2 GiB input).  Algorithmic bytes as
    in the step (2 B read + 1 B written per element + 4 B per scale).  The
    headline entries are the 32768^2 ones; below 8192^2 the calls are
    launch-bound, and those sizes are also timed replayed from a HIP graph
    (graph_avg_us), which leaves out the host's per-call cost."""
    from synth import inputs
    dev = torch.device("cuda", 0)
    sweep = {}
    for size in sizes:
        nbuf = max(1, cdiv(rotate_bytes, 2 * size * size))
        x0 = inputs.randn_bf16((size, size), seed=inputs.tensor_seed(seed, "a"), device=dev)
        xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
        qs = [torch.empty(size, size, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        entry = {"buffers": nbuf}
        for block in ("1x128", "128x128"):
            nkb = cdiv(size, 128)
            rows = size if block == "1x128" else cdiv(size, 128)
            recips = [torch.empty(nkb, rows, dtype=torch.float32, device=dev).t() for _ in range(nbuf)]
            ms = _time_quant(xs, qs, recips, block, reps)
            gbps = quant_bytes(size, size, block) / (ms * 1e-3) / 1e9
            entry[block] = {"avg_us": round(ms * 1e3, 2), "gbps": round(gbps, 1),
                            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBS, 4)}
            if size < 8192:
                # launch-bound sizes: the same calls replayed from a HIP graph
                gms = _time_quant(xs, qs, recips, block, reps, graph=True)
                entry[block]["graph_avg_us"] = round(gms * 1e3, 2)
                entry[block]["graph_gbps"] = round(quant_bytes(size, size, block) / (gms * 1e-3) / 1e9, 1)
            del recips
        sweep[str(size)] = entry
        del xs, qs, x0
        torch.cuda.empty_cache()
    top = sweep[str(max(sizes))]
    return {"shape": [max(sizes), max(sizes)], "1x128": top["1x128"], "128x128": top["128x128"],
            "sweep": sweep}


def grouped_gemm(seed, wl, groups=8, reps=10):
    """The grouped (mixture-of-experts) blockwise GEMM at the forward shape:
    the M = 16640 quantized tokens of X split over `groups` experts with
    seeded multinomial sizes, one 128x128-quantized N x K weight per expert;
    2MNK flops in total, timed with a HIP event pair around `reps` calls
    after at least 0.5 s of warm-up calls."""
    import numpy as np
    import blockwise_scaled_fp8_amd as fp8
    from synth import inputs
    dev = torch.device("cuda", 0)
    wq = torch.empty(groups, N, K, dtype=torch.uint8, device=dev)
    wr = torch.empty(groups, cdiv(K, 128), cdiv(N, 128), dtype=torch.float32, device=dev).transpose(1, 2)
    for g in range(groups):
        w = inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(seed + 100 + g, "w"), device=dev)
        fp8.fp8_blockwise_quant(w, "128x128", q=wq[g], recip=wr[g])
        del w
    sizes = np.random.default_rng(seed).multinomial(M, np.ones(groups) / groups)
    ends = torch.tensor(np.cumsum(sizes), dtype=torch.int32, device=dev)
    out = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    call = lambda: fp8.fp8_scaled_grouped_gemm_blockwise(wl.xq, wl.xr, wq, wr, ends, out=out)  # noqa: E731
    ms = _event_avg_ms(call, reps, warm_s=0.5)
    tflops = 2 * M * N * K / (ms * 1e-3) / 1e12
    return {"groups": groups, "group_rows": [int(v) for v in sizes], "M": M, "N": N, "K": K,
            "avg_us": round(ms * 1e3, 1), "tflops": round(tflops, 1),
            "frac_of_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
            "launches": "whole 256x256 row tiles of every expert (and last tiles of more than "
                        "128 rows), then the experts' smaller last tiles as 64x64 tiles when that "
                        "saves a round of the CUs"}


def _event_avg_ms(call, reps, warm=3, warm_s=0.0):
    """Average duration (ms) of `call` over `reps` back-to-back calls on
    torch's current stream (the stream the library launches on), from one
    HIP event pair around the whole run.  Warm-up: `warm` calls, then more
    until `warm_s` seconds have passed (the shader clock settles at its
    loaded level within a few hundred ms of sustained MFMA work)."""
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < warm_s:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _graph_avg_ms(call, reps):
    """The same calls captured once as a HIP graph and replayed (the host's
    per-call cost drops out)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            call()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _gemm_entry(ms, flop):
    t = flop / (ms * 1e-3) / 1e12
    return {"avg_us": round(ms * 1e3, 2), "tflops": round(t, 2),
            "frac_of_fp8_peak": round(t / FP8_PEAK_TFLOPS, 4)}


def _quant_entry(ms, nbytes):
    g = nbytes / (ms * 1e-3) / 1e9
    return {"avg_us": round(ms * 1e3, 2), "gbps": round(g, 1),
            "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4)}


def tiny_linear(seed, reps=200):
    """The tiny linear: X [128, 512] N(0,1), W [256, 512] nn.Linear init, dY
    [128, 256]; the fused training step (quantization included) and its
    forward GEMM alone, eager and replayed from a HIP graph.  Latency-bound:
    2MNK = 3.4e7 flops per GEMM."""
    import blockwise_scaled_fp8_amd as fp8
    dev = torch.device("cuda", 0)
    shape = (128, 256, 512)
    wl = Workload(seed, dev, shape)
    plan = step_plan_dual(wl)
    m, n, k = shape

    def step():
        for _, fn, _, _ in plan:
            fn()
    gemm = lambda: fp8.fp8_scaled_gemm_blockwise(wl.xq, wl.xr, wl.wq, wl.wr, "128x128", out=wl.y)  # noqa: E731
    step()
    ms = _event_avg_ms(step, reps)
    gms = _graph_avg_ms(step, reps)
    flop = 3 * 2 * m * n * k
    return {"M": m, "N": n, "K": k, "plan": fp8.gemm_plan(m, n, k),
            "step": {"launches": len(plan), "avg_us": round(ms * 1e3, 2),
                     "graph_avg_us": round(gms * 1e3, 2),
                     "graph_tflops": round(flop / (gms * 1e-3) / 1e12, 3)},
            "gemm_fwd": dict(_gemm_entry(_event_avg_ms(gemm, reps), 2 * m * n * k),
                             graph_avg_us=round(_graph_avg_ms(gemm, reps) * 1e3, 2))}


def per_tensor(seed, reps=200):
    """Per-tensor FP8: X [256, 1024] and W [4096, 1024] N(0,1) bf16, each
    quantized with one scale (two launches: partial amax, then quantize;
    5 B moved per element, 3 B algorithmic), and the tensorwise GEMM
    256 x 4096 x 1024 with bf16 out; the 16 x 32 x 32 fp32-out edge case the
    same way.  Both are latency-bound; graph-replayed times leave out the
    host's per-call cost."""
    import blockwise_scaled_fp8_amd as fp8
    from synth import inputs
    dev = torch.device("cuda", 0)
    out = {}
    for (m, n, k), od in (((256, 4096, 1024), torch.bfloat16), ((16, 32, 32), torch.float32)):
        x = inputs.randn_bf16((m, k), seed=inputs.tensor_seed(seed + 30, "x"), device=dev)
        w = inputs.randn_bf16((n, k), seed=inputs.tensor_seed(seed + 30, "w"), device=dev)
        xq, xr = fp8.fp8_tensorwise_quant(x)
        wq, wr = fp8.fp8_tensorwise_quant(w)
        y = torch.empty(m, n, dtype=od, device=dev)
        qx = lambda: fp8.fp8_tensorwise_quant(x, q=xq, recip=xr)  # noqa: E731
        qw = lambda: fp8.fp8_tensorwise_quant(w, q=wq, recip=wr)  # noqa: E731
        g = lambda: fp8.fp8_scaled_gemm_tensorwise(xq, xr, wq, wr, out=y)  # noqa: E731
        e = {}
        for name, fn, elems in (("quant X", qx, m * k), ("quant W", qw, n * k)):
            ms, gms = _event_avg_ms(fn, reps), _graph_avg_ms(fn, reps)
            e[name] = {"avg_us": round(ms * 1e3, 2), "graph_avg_us": round(gms * 1e3, 2),
                       "graph_gbps_moved_5B": round(5 * elems / (gms * 1e-3) / 1e9, 1),
                       "graph_gbps_algorithmic_3B": round(3 * elems / (gms * 1e-3) / 1e9, 1)}
        e["gemm"] = dict(_gemm_entry(_event_avg_ms(g, reps), 2 * m * n * k),
                         graph_avg_us=round(_graph_avg_ms(g, reps) * 1e3, 2))
        e["gemm"]["graph_tflops"] = round(2 * m * n * k / (e["gemm"]["graph_avg_us"] * 1e-6) / 1e12, 2)
        e["out"] = "bf16" if od == torch.bfloat16 else "fp32"
        out[f"{m}x{n}x{k}"] = e
    return out


def tensorwise_quant_large(seed, sizes=(8192, 16384, 32768), reps=5):
    """The per-tensor quantizer on S x S bf16 (inputs rotated over at least
    1 GiB like the blockwise sweep): one amax pass (2 B read per element)
    and one quantize pass (2 B read + 1 B written), so 5 B move per element
    against 3 B algorithmic; both rates reported."""
    import blockwise_scaled_fp8_amd as fp8
    from synth import inputs
    dev = torch.device("cuda", 0)
    res = {}
    for size in sizes:
        nbuf = max(1, cdiv(1 << 30, 2 * size * size))
        x0 = inputs.randn_bf16((size, size), seed=inputs.tensor_seed(seed, "a"), device=dev)
        xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
        qs = [torch.empty(size, size, dtype=torch.uint8, device=dev) for _ in range(nbuf)]
        rs = [torch.empty(1, dtype=torch.float32, device=dev) for _ in range(nbuf)]
        calls = max(reps, 2 * nbuf)
        it = {"i": 0}

        def call():
            i = it["i"] % nbuf
            it["i"] += 1
            fp8.fp8_tensorwise_quant(xs[i], q=qs[i], recip=rs[i])
        ms = _event_avg_ms(call, calls)
        e = size * size
        res[str(size)] = {"buffers": nbuf, "avg_us": round(ms * 1e3, 2),
                          "gbps_moved_5B": round(5 * e / (ms * 1e-3) / 1e9, 1),
                          "frac_of_hbm_peak_moved": round(5 * e / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "gbps_algorithmic_3B": round(3 * e / (ms * 1e-3) / 1e9, 1),
                          "frac_of_hbm_peak_algorithmic": round(3 * e / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del xs, qs, rs, x0
        torch.cuda.empty_cache()
    return res


def long_k(seed, reps=10):
    """The long-K blockwise GEMM: M = N = 1024, K = 128000 / 128128 / 128256
    (1000 / 1001 / 1002 K blocks); A N(0,1) 1x128, B nn.Linear init
    128x128, bf16 out.  The whole call (split-K main launch plus the ordered
    reduce) per 2MNK flops; the quantizers of A and B are timed too."""
    import blockwise_scaled_fp8_amd as fp8
    from synth import inputs
    dev = torch.device("cuda", 0)
    m = n = 1024
    res = {}
    for k in (128000, 128128, 128256):
        a = inputs.randn_bf16((m, k), seed=inputs.tensor_seed(seed + 20, "a"), device=dev)
        b = inputs.linear_weight_bf16(n, k, seed=inputs.tensor_seed(seed + 20, "b"), device=dev)
        aq, ar = fp8.fp8_blockwise_quant(a, "1x128")
        bq, br = fp8.fp8_blockwise_quant(b, "128x128")
        y = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        ms = _event_avg_ms(lambda: fp8.fp8_scaled_gemm_blockwise(aq, ar, bq, br, "128x128", out=y),
                           reps, warm_s=0.3)
        qa = _event_avg_ms(lambda: fp8.fp8_blockwise_quant(a, "1x128", q=aq, recip=ar), reps)
        qb = _event_avg_ms(lambda: fp8.fp8_blockwise_quant(b, "128x128", q=bq, recip=br), reps)
        res[str(k)] = {"k_blocks": k // 128, "plan": fp8.gemm_plan(m, n, k),
                       "gemm": _gemm_entry(ms, 2 * m * n * k),
                       "quant_1x128 A": _quant_entry(qa, quant_bytes(m, k, "1x128")),
                       "quant_128x128 B": _quant_entry(qb, quant_bytes(n, k, "128x128"))}
        del a, b, aq, bq, y
        torch.cuda.empty_cache()
    return res


def cpu_baseline(seed, min_seconds=10.0, max_samples=8):
    """The oracle, as it stands, on a bounded sample of the same workload.
    One sample: fwd and dgrad on 64 output rows (each with the full quantized
    weight) and wgrad on 64 x 1024 outputs (full M contraction), inputs drawn
    on the host with the same recipe.  Fresh samples (new seeds) are run
    until at least `min_seconds` of oracle time has accumulated (at most
    `max_samples`), and the rate is total sampled flops / total time."""
    from oracle import linear
    from synth import inputs
    rows, kcols = 64, 1024
    g = inputs.bf16_bits
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        pass
    flops_one = 2 * rows * N * K + 2 * rows * K * N + 2 * rows * kcols * M
    total_t, n = 0.0, 0
    while n < max_samples and (n == 0 or total_t < min_seconds):
        sd = seed + 1000 * (n + 1)
        x = g(inputs.randn_bf16((rows, K), seed=inputs.tensor_seed(sd, "x")))
        w = g(inputs.linear_weight_bf16(N, K, seed=inputs.tensor_seed(sd, "w")))
        dy = g(inputs.randn_bf16((rows, N), seed=inputs.tensor_seed(sd, "dy")))
        dy_cols = g(inputs.randn_bf16((M, rows), seed=inputs.tensor_seed(sd + 1, "dy")))
        x_cols = g(inputs.randn_bf16((M, kcols), seed=inputs.tensor_seed(sd + 1, "x")))
        t0 = time.perf_counter()
        linear.fwd(x, w)
        linear.dgrad(dy, w)
        linear.wgrad(dy_cols, x_cols)
        total_t += time.perf_counter() - t0
        n += 1
    flops = flops_one * n
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(flops / total_t / 1e12, 6), "unit": "TFLOP/s",
            "cores": threads or len(os.sched_getaffinity(0)), "kind": "oracle",
            "host": {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                     "torch_threads": torch.get_num_threads(), "blas_threads": threads,
                     "cpu_model": model},
            "sample": (f"{n} samples, each the oracle (quantize + block-rescaled float64 GEMM) "
                       f"for fwd and dgrad on {rows} of {M} output rows and wgrad on {rows} x "
                       f"{kcols} of {N} x {K} outputs (full contraction, full quantization of "
                       f"each operand used): {flops / 1e9:.1f} GFLOP in {total_t:.1f} s")}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "linear_step_M16640_N5120_K8192_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "blockwise_scaled_fp8_amd", "csrc", "gemm.hip")


def measured_traffic(call):
    """HBM bytes of one GEMM call of the step ("gemm fwd" / "gemm dgrad" /
    "gemm wgrad", all its launches), from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary, valid only while the GEMM source is the
    one those counters were taken on (sha256 recorded in the summary)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
        rec = json.loads(text.split("TRAFFIC_JSON:", 1)[1].strip().splitlines()[0])
        sha = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except (OSError, IndexError, ValueError):
        return None
    if rec.get("gemm_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_call", {}).get(call)


def gemm_plans(shape=(M, N, K)):
    """The launches of each GEMM call of the step (main launch, then the
    leftover tiles' K split and reduce where the plan has them), from the
    library's plan for this device."""
    import blockwise_scaled_fp8_amd as fp8
    m, n, k = shape
    out = {}
    for nm, (gm, gn, gk, mode) in (("gemm fwd", (m, n, k, "128x128")),
                                   ("gemm dgrad", (m, k, n, "128x128")),
                                   ("gemm wgrad", (n, k, m, "1x128"))):
        pl = fp8.gemm_plan(gm, gn, gk, mode)
        nmain = pl['tiles_full'] if pl['tail_splits'] > 1 else pl['tiles']
        ntail = pl['tiles'] - pl['tiles_full']
        parts = [f"main launch {nmain} tiles"]
        # The library runs two or more full rounds of interior 256x256 tiles
        # (bf16 out, contiguous rows) as a persistent launch, the leftover
        # tiles' K pieces included.
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        persist = (pl["config"] == 3 and pl["splits"] == 1 and gm % 256 == 0 and gn % 256 == 0
                   and nmain >= 2 * cus and nmain % cus == 0
                   and (pl["tail_splits"] <= 1 or ntail * pl["tail_splits"] <= cus))
        if persist:
            parts[0] += f" ({cus} persistent workgroups x {nmain // cus}"
            if pl["tail_splits"] > 1:
                parts[0] += f", then {ntail} leftover tiles x {pl['tail_splits']} K pieces"
            parts[0] += ")"
        if pl["splits"] > 1:
            parts[0] += f" x {pl['splits']} K splits"
            parts.append("ordered reduce")
        if pl["tail_splits"] > 1:
            if not persist:
                parts.append(f"{ntail} leftover tiles x {pl['tail_splits']} K splits")
            parts.append("ordered reduce")
        out[nm] = dict(pl, launches=" + ".join(parts))
    return out


def copy_probe(gib):
    """A plain device-to-device copy of `gib` GiB (one read + one write of
    each byte), run so that a profiler's FETCH_SIZE / WRITE_SIZE for it can
    calibrate the same counters on the GEMM."""
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quant-standalone", action="store_true",
                    help="skip the standalone quantizer sweep (S x S, S = 1024 .. 32768)")
    ap.add_argument("--step-only", action="store_true",
                    help="time the step alone: no separate-quantizer step, second linear shape, "
                         "grouped GEMM or standalone quantizers (for profiling runs)")
    ap.add_argument("--copy-probe-gib", type=float, default=0.0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--only", choices=["long_k"], default=None,
                    help="run this one other workload alone and print its record (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the hot path runs "
              "on a single MI355X; sharding it across GPUs is described, not measured.",
              file=sys.stderr)
        sys.exit(2)
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs as a single process on one GPU", file=sys.stderr)
        sys.exit(2)

    if args.only == "long_k":
        print(json.dumps({"long_k": long_k(args.seed)}), flush=True)
        return
    r = run_gpu(args.steps, args.warmup, args.seed, plan_fn=step_plan_dual)
    step_ms = r["gpu_ms_per_step"]
    flops = 3 * 2 * M * N * K
    value = flops / (step_ms * 1e-3) / 1e12
    names = [p[0] for p in r["plan"]]
    rooflines = {}
    for nm in ("gemm fwd", "gemm dgrad", "gemm wgrad"):
        ms = r["per_ms"][names.index(nm)]
        ach = 2 * M * N * K / (ms * 1e-3) / 1e12
        rooflines[nm] = {"bound": "mfma", "avg_us": round(ms * 1e3, 2),
                         "flop_per_call": 2 * M * N * K, "achieved": round(ach, 1),
                         "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(ach / FP8_PEAK_TFLOPS, 4),
                         "share_of_step": round(ms / r["gpu_ms_per_step_with_call_events"], 4)}
    dominant = max(rooflines, key=lambda k: rooflines[k]["avg_us"])
    dom = rooflines[dominant]
    plans = gemm_plans()
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic: X, dY ~ N(0,1) bf16; W ~ U(+-1/sqrt(K)) bf16 (nn.Linear init); seeded",
        "config": {"workload": "fp8 blockwise linear fwd+dgrad+wgrad incl. quantization",
                   "M": M, "N": N, "K": K, "recipes": "fwd/dgrad 1x128 x 128x128, wgrad 1x128 x 1x128",
                   "quantization": "fused: X and dY each read once into both code layouts; "
                                   "W into W codes in the forward and W^T codes right before dgrad",
                   "seed": args.seed},
        "roofline": {"bound": "mfma",
                     "kernel": f"{dominant.split()[1]} blockwise GEMM call "
                               f"({plans[dominant]['launches']})",
                     "achieved": dom["achieved"], "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": dom["frac"], "traffic": measured_traffic(dominant)},
        "rooflines": {k: dict(v, launches=plans[k]["launches"]) for k, v in rooflines.items()},
        "gemm_tflops": {k: v["tflops"] for k, v in r["kernels"].items() if "tflops" in v},
        "quant_gbps": round(r["quant_gbps"], 1),
        "quant_frac_of_hbm_peak": round(r["quant_gbps"] / HBM_PEAK_GBS, 4),
        "quant_note": "the four quantizer launches of the step (X and dY into both code layouts "
                      "from one read, W into W and, in the backward, into W^T): algorithmic bytes "
                      "(bf16 read, codes and scales written) / their event time",
        "kernels": r["kernels"],
        "wall_ms_per_step": round(r["wall_ms_per_step"], 4),
        "ms_per_step_with_call_events": round(r["gpu_ms_per_step_with_call_events"], 4),
    }
    if args.step_only:
        args.no_quant_standalone = True
    rd = (None if args.step_only else
          run_gpu(args.steps, args.warmup, args.seed, plan_fn=step_plan, wl=r["workload"]))
    if rd is not None:
        out["separate_quant_step"] = {
            "note": "same step with six separate quantizer launches (X and dY each read twice)",
            "ms_per_step": round(rd["gpu_ms_per_step"], 4),
            "value": round(flops / (rd["gpu_ms_per_step"] * 1e-3) / 1e12, 1),
            "quant_us_per_step": round(rd["quant_us"], 1),
            "quant_gbps": round(rd["quant_gbps"], 1),
            "kernels": rd["kernels"]}
        out["grouped_gemm"] = grouped_gemm(args.seed, r["workload"])
    del r, rd
    if not args.step_only:
        # the second linear shape of the workload (N and K swapped)
        r2 = run_gpu(args.steps, args.warmup, args.seed, plan_fn=step_plan_dual, shape=SHAPE2)
        m2, n2, k2 = SHAPE2
        out["step_%dx%dx%d" % SHAPE2] = {
            "M": m2, "N": n2, "K": k2,
            "ms_per_step": round(r2["gpu_ms_per_step"], 4),
            "value": round(3 * 2 * m2 * n2 * k2 / (r2["gpu_ms_per_step"] * 1e-3) / 1e12, 1),
            "gemm_tflops": {k: v["tflops"] for k, v in r2["kernels"].items() if "tflops" in v},
            "quant_gbps": round(r2["quant_gbps"], 1)}
        del r2
    if not args.no_quant_standalone:
        out["quant_standalone"] = quant_standalone(args.seed)
    if not args.step_only:
        out["tiny_linear"] = tiny_linear(args.seed)
        out["per_tensor"] = per_tensor(args.seed)
        out["tensorwise_quant"] = tensorwise_quant_large(args.seed)
        out["long_k"] = long_k(args.seed)
    if args.copy_probe_gib > 0:
        out["copy_probe_bytes"] = copy_probe(args.copy_probe_gib)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.seed)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
