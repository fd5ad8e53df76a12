#!/usr/bin/env python3
"""Benchmark of the delayed-scaling FP8 hot path on one MI355X.

One step = one pass of the path over one batch of synthetic input, the
square 8192^3 workload: delayed-scaling quantize of A [8192, 8192] and of
B [8192, 8192] (bf16 ~ N(0,1), E4M3, history 16, amax + ring update fused)
followed by the scaled FP8 GEMM C = A8 * B8^T (NT, fp32 accumulate, bf16
out).  Inputs are resident in HBM before timing starts; three copies of the
inputs rotate so the 256 MB Infinity Cache cannot serve a step from the
previous one.

Prints one JSON line.  `value` is the step's GEMM FLOPs over the measured
step time (both quantizes included), in TFLOP/s.  `roofline` is the GEMM
kernel's own rate (HIP events around each launch, on the launch stream)
against the dense FP8 MFMA peak; `roofline_quantize` the quantize kernel's
against HBM.  After the W warm-up steps the step runs untimed for
--settle-ms more (the clocks ramp for tens of milliseconds under this load);
`clock_settle` reports how long and how many steps.  `configs` times every
other workload of the path (the linear layer's GEMMs and quantizes, the
square sweep, the skinny and batched GEMMs, the 12-layer chain at 4096
tokens) against its roofline, and `per_linear_overhead` the fixed cost of one
FP8 linear layer.  `cpu_baseline` times the oracle (numpy) on bounded slices
of the same work on the host.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA, published
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--size", type=int, default=8192, help="M = N = K of the square workload")
    ap.add_argument("--rotate", type=int, default=3, help="input copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-rows", type=int, default=256, help="output rows of the oracle sample")
    ap.add_argument("--no-widened", action="store_true", help="skip the widened-path kernel timings")
    ap.add_argument("--no-linear-step", action="store_true", help="skip the 12-layer linear step")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config timings")
    ap.add_argument("--only-config", default=None,
                    choices=["linear_d1024_t2048", "square_sweep", "skinny_batched", "chain_12_layers_t4096"],
                    help="time one group of the per-config workloads only (nothing else) and print it")
    ap.add_argument("--settle-ms", type=float, default=400.0,
                    help="untimed steps after the warm-up, in milliseconds, before the timed steps")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "delayed_scaling_amd", "csrc")
# Device sources of each kernel family: the recorded HBM traffic holds only
# while their hash is the one it was measured with.
GEMM_SOURCES = [os.path.join(CSRC, f) for f in ("gemm_kernel.h", "gemm.hip", "device_common.h")]
QUANT_SOURCES = [os.path.join(CSRC, f) for f in ("quantize.hip", "device_common.h")]


def sources_sha(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def traffic_from_profile(kernel_srcs, sha_key, bytes_key):
    """HBM bytes per launch recorded in profiles/ by the two PMC runs, or
    None when the kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_8192_bench_kernels.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = sources_sha(kernel_srcs)
    m_sha = re.search(rf"^{sha_key}:\s*([0-9a-f]{{64}})", text, re.M)
    m_b = re.search(rf"^{bytes_key}:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def cpu_baseline(a_bits, b_bits, size, rows):
    """The oracle as it stands, timed on the host on bounded slices of the
    benchmark's work (about 10-20 s in all):
      * value: the headline step on its first `rows` output rows (quantize all
        of B and `rows` rows of A, then the fp64 GEMM of the slice), as GEMM
        FLOPs of the slice per second, the matmul on all BLAS threads;
      * one_thread: the same GEMM slice (an eighth of the rows) on one thread;
      * quantize_gbps: the delayed-scaling quantize of 2048 rows of A
        (bytes moved: 2 read + 1 written per element), numpy on one thread;
      * per_config: the oracle's quantize + GEMM of the square 1024^3 and of
        the linear layer's forward (2048x4096x1024), all BLAS threads."""
    import numpy as np
    import threadpoolctl

    import oracle
    info = threadpoolctl.threadpool_info()
    blas_threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    t0 = time.perf_counter()
    ra = oracle.ring_init(16, oracle.E4M3)
    rb = oracle.ring_init(16, oracle.E4M3)
    qa, ra = oracle.quantize_step(ra, a_bits[:rows])
    qb, rb = oracle.quantize_step(rb, b_bits)
    oracle.mm(qa.reshape(-1), qb.reshape(-1), 0, 0, oracle.NT, rows, size, size, size, size,
              ra.scale_inv_used, rb.scale_inv_used)
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * size * size

    r1 = max(1, rows // 8)
    with threadpoolctl.threadpool_limits(limits=1, user_api="blas"):
        t1 = time.perf_counter()
        oracle.mm(qa[:r1].reshape(-1), qb.reshape(-1), 0, 0, oracle.NT, r1, size, size, size, size,
                  ra.scale_inv_used, rb.scale_inv_used)
        dt1 = time.perf_counter() - t1
    qrows = min(2048, size)
    t2 = time.perf_counter()
    oracle.quantize_step(oracle.ring_init(16, oracle.E4M3), a_bits[:qrows])
    dtq = time.perf_counter() - t2

    def config(m, n, k):
        from synth import bf16_normal
        x, w = bf16_normal((m, k), 11), bf16_normal((n, k), 12)
        t = time.perf_counter()
        cx, rx = oracle.quantize_step(oracle.ring_init(16, oracle.E4M3), x)
        cw, rw = oracle.quantize_step(oracle.ring_init(16, oracle.E4M3), w)
        oracle.mm(cx.reshape(-1), cw.reshape(-1), 0, 0, oracle.NT, m, n, k, k, k, rx.scale_inv_used,
                  rw.scale_inv_used)
        d = time.perf_counter() - t
        return {"seconds": round(d, 3), "tflops": round(2.0 * m * n * k / d / 1e12, 6),
                "work": f"quantize {m}x{k} and {n}x{k}, fp64 GEMM {m}x{n}x{k}"}

    per_config = {"square_1024": config(1024, 1024, 1024), "linear_fwd_2048x4096x1024": config(2048, 4096, 1024)}
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": (f"first {rows} of {size} output rows: quantize B ({size}x{size}) and {rows} rows of A, "
                       f"fp64 GEMM of the slice; {dt:.1f} s; numpy elementwise steps on 1 thread, "
                       f"the fp64 matmul on {blas_threads} BLAS threads"),
            "one_thread": {"value": round(2.0 * r1 * size * size / dt1 / 1e12, 6), "unit": "TFLOP/s",
                           "sample": f"fp64 GEMM of {r1} output rows on 1 BLAS thread, {dt1:.1f} s"},
            "quantize_gbps": {"value": round(3.0 * qrows * size / dtq / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "sample": f"quantize {qrows}x{size} bf16 -> E4M3 with its ring, {dtq:.1f} s"},
            "per_config": per_config}


def time_launches(fn, stream, reps=12, warmup=3):
    """Average duration of fn(i) in microseconds: HIP events on the launch
    stream around `reps` back-to-back calls, after `warmup` calls.  i counts
    the calls, so fn can rotate over input copies."""
    import torch
    for i in range(warmup):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def measure_widened(ds, n, stream, rot=3):
    """Rooflines of the path's other kernels on n x n operands: the single-
    tensor quantize, the transposed and dual quantize, the dynamic recipe
    (amax pass + quantize), fp32 and fp16 inputs, the bias gradient of an
    n x n gradient, and the dX / dW GEMM layouts in the backward formats
    (E5M2 x E4M3).  Every launch takes the next of `rot` input and output
    copies, so the 256 MB Infinity Cache cannot carry one launch's data into
    the next."""
    import torch
    from synth import bf16_normal, seed_for
    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(bf16_normal((n, n), seed_for(3, 0, "X")).view("int16")).view(torch.bfloat16).to(dev)
    X = [x0] + [x0.clone() for _ in range(rot - 1)]
    Y = [torch.empty((n, n), dtype=torch.uint8, device=dev) for _ in range(rot)]
    YT = [torch.empty((n, n), dtype=torch.uint8, device=dev) for _ in range(rot)]
    ring = ds.ScaleRing(16, ds.E4M3)
    ring1 = ds.ScaleRing(1, ds.E4M3)
    out = {}

    def hbm(name, us, nbytes, workload):
        gbps = nbytes / (us * 1e-6) / 1e9
        out[name] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "avg_launch_us": round(us, 2),
                     "bytes_per_launch": nbytes, "workload": workload}

    us = time_launches(lambda i: ds.fp8_quantize(X[i % rot], ds.E4M3, ring, out=Y[i % rot]), stream)
    hbm("quantize_single", us, 3.0 * n * n, f"{n}x{n} bf16 -> E4M3, history 16, one tensor per launch")
    us = time_launches(lambda i: ds.fp8_quantize_2d(X[i % rot], ds.E4M3, ring, ds.TRANSPOSED, out_t=YT[i % rot]),
                       stream)
    hbm("quantize_2d_transposed", us, 3.0 * n * n, f"{n}x{n} bf16 -> E4M3 codes of x^T, history 16")
    us = time_launches(lambda i: ds.fp8_quantize_2d(X[i % rot], ds.E4M3, ring, ds.DUAL, out=Y[i % rot],
                                                    out_t=YT[i % rot]), stream)
    hbm("quantize_2d_dual", us, 4.0 * n * n, f"{n}x{n} bf16 -> E4M3 codes of x and x^T, history 16")
    us = time_launches(lambda i: ds.fp8_quantize_dynamic(X[i % rot], ds.E4M3, ring1, out=Y[i % rot]), stream)
    hbm("quantize_dynamic", us, 5.0 * n * n, f"{n}x{n} bf16, amax pass + quantize pass (two launches)")
    x16 = [x.half() for x in X]
    us = time_launches(lambda i: ds.fp8_quantize(x16[i % rot], ds.E4M3, ring, out=Y[i % rot]), stream)
    hbm("quantize_fp16_input", us, 3.0 * n * n, f"{n}x{n} fp16 -> E4M3, history 16")
    del x16
    x32 = [x.float() for x in X]
    us = time_launches(lambda i: ds.fp8_quantize(x32[i % rot], ds.E4M3, ring, out=Y[i % rot]), stream)
    hbm("quantize_fp32_input", us, 5.0 * n * n, f"{n}x{n} fp32 -> E4M3, history 16")
    del x32
    ws = ds.BiasGradWorkspace(n, n)
    gb = torch.empty(n, dtype=torch.bfloat16, device=dev)
    us = time_launches(lambda i: ds.fp8_bias_grad(X[i % rot], out=gb, workspace=ws), stream)
    hbm("bias_grad", us, 2.0 * n * n + 2.0 * n, f"column sums of a {n}x{n} bf16 gradient, bf16 out")
    del X, Y, YT
    a8 = [torch.randint(0, 120, (n, n), dtype=torch.uint8, device=dev) for _ in range(rot)]
    b8 = [torch.randint(0, 120, (n, n), dtype=torch.uint8, device=dev) for _ in range(rot)]
    c = [torch.empty((n, n), dtype=torch.bfloat16, device=dev) for _ in range(rot)]
    for name, layout in (("gemm_nn_dx", ds.NN), ("gemm_tn_dw", ds.TN)):
        # 40 untimed launches (about 20 ms) first: after the memory-bound kernels
        # above, the clocks take that long to settle under the MFMA load.
        us = time_launches(lambda i: ds.fp8_mm(a8[i % rot], b8[i % rot], ds.E5M2, ds.E4M3, layout, n, n, n, ring,
                                               ring, out=c[i % rot]), stream, warmup=40)
        tf = 2.0 * n ** 3 / (us * 1e-6) / 1e12
        out[name] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_FP8_TFLOPS, 4), "avg_launch_us": round(us, 2),
                     "workload": f"{n}^3 {'NN' if layout == ds.NN else 'TN'} E5M2 x E4M3, bf16 out"}
    return out


def measure_linear_step(stream, tokens=2048, dim=1024, layers=12, steps=5):
    """Forward + backward of the linear layers of a 12-layer, dim-1024 model on
    `tokens` tokens (per layer QKV 1024->3072, O 1024->1024, MLP up 1024->4096
    and down 4096->1024, no bias): the library's FP8 layer against torch's bf16
    linear, each linear with its own synthetic input and output gradient.
    Every step starts with the gradients unset, as after an optimizer's
    zero_grad(set_to_none=True), so backward writes them without an add."""
    import torch
    from delayed_scaling_amd.linear import Fp8Linear
    shapes = [(dim, 3 * dim), (dim, dim), (dim, 4 * dim), (4 * dim, dim)] * layers
    gen = torch.Generator("cuda").manual_seed(4000)
    xs = [torch.randn(tokens, i, device="cuda", generator=gen).to(torch.bfloat16).requires_grad_() for i, _ in shapes]
    gs = [(torch.randn(tokens, o, device="cuda", generator=gen) * 1e-3).to(torch.bfloat16) for _, o in shapes]
    fp8 = [Fp8Linear(i, o, bias=False) for i, o in shapes]
    bf16 = [torch.nn.Linear(i, o, bias=False, device="cuda", dtype=torch.bfloat16) for i, o in shapes]

    def run(mods):
        for m, x, g in zip(mods, xs, gs):
            x.grad = None                      # as an optimizer's zero_grad(set_to_none=True)
            m.weight.grad = None
            m(x).backward(g)

    def timed(fn):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {}
    # Eager steps are bound by host time, which drifts while the process
    # runs: the two paths alternate over three rounds, and each reports the
    # mean of its rounds.
    for name, mods in (("fp8", fp8), ("bf16", bf16)):
        for _ in range(3):
            run(mods)
    eager = {"fp8": [], "bf16": []}
    for _ in range(3):
        for name, mods in (("fp8", fp8), ("bf16", bf16)):
            eager[name].append(timed(lambda: run(mods)))
    for name in eager:
        res[name + "_eager"] = sum(eager[name]) / len(eager[name])
    for name, mods in (("fp8", fp8), ("bf16", bf16)):
        # The same step captured once in a HIP graph and replayed: no host work per call.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run(mods)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run(mods)
        graph.replay()
        res[name] = timed(graph.replay)
    flops = 6.0 * tokens * sum(i * o for i, o in shapes)
    return {"workload": f"{layers} layers x 4 linears (dim {dim}, {tokens} tokens), forward + backward, no bias, "
                        "gradients set to None before each step, each step captured in a HIP graph",
            "fp8_ms_per_step": round(res["fp8"], 3), "bf16_ms_per_step": round(res["bf16"], 3),
            "speedup_vs_bf16": round(res["bf16"] / res["fp8"], 3),
            "fp8_tflops": round(flops / (res["fp8"] * 1e-3) / 1e12, 1),
            "bf16_tflops": round(flops / (res["bf16"] * 1e-3) / 1e12, 1),
            "eager_fp8_ms_per_step": round(res["fp8_eager"], 3), "eager_bf16_ms_per_step": round(res["bf16_eager"], 3),
            "eager_rounds_ms": {k: [round(v, 3) for v in eager[k]] for k in eager},
            "gemm_flops": flops}


def spread_us(ms_list):
    """p10 / median / p90 of per-launch times given in milliseconds, in microseconds."""
    v = sorted(ms_list)
    pick = lambda f: round(v[min(len(v) - 1, int(f * len(v)))] * 1e3, 2)
    return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}


def time_each(fn, stream, reps, warmup):
    """Per-launch durations (milliseconds) of fn(i): a HIP event before and
    after every call on the launch stream, after `warmup` untimed calls."""
    import torch
    for i in range(warmup):
        fn(i)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        fn(warmup + i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]


def gemm_entry(ms, m, n, k, batch, nbytes, workload):
    """A GEMM timing against its roofline: the dense FP8 MFMA peak and the HBM
    bound of its algorithmic bytes (A + B + C + bias once each); `attainable`
    is min(peak, bytes-bound rate) and `frac` the achieved share of it."""
    us = spread_us(ms)["p50"]
    flops = 2.0 * m * n * k * batch
    tf = flops / (us * 1e-6) / 1e12
    gbps = nbytes / (us * 1e-6) / 1e9
    attain = min(PEAK_FP8_TFLOPS, flops / nbytes * PEAK_HBM_GBPS / 1e3)
    return {"workload": workload, "us_p50": us, "launch_us": spread_us(ms), "tflops": round(tf, 1),
            "gbps": round(gbps, 1), "frac_mfma": round(tf / PEAK_FP8_TFLOPS, 4),
            "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
            "bound": "mfma" if attain >= PEAK_FP8_TFLOPS else "hbm",
            "roofline_us": round(flops / (attain * 1e12) * 1e6, 2), "frac": round(tf / attain, 4),
            "flops": flops, "bytes": nbytes}


def measure_configs(ds, stream, only=None):
    """Every workload of the path besides the 8192^3 headline, each timed on
    its own (per-launch HIP events, median of 60-100 launches after warm-up)
    with inputs rotated over enough copies to exceed the 256 MB Infinity
    Cache where the work is HBM-bound:
      * the linear layer at dim 1024, 2048 tokens: forward NT
        2048x4096x1024 with a bf16 bias, dX NN 2048x1024x4096 and dW TN
        4096x1024x2048 (E5M2 x E4M3), and the quantizes of X, W and G;
      * the square sweep at 1024, 2048 and 4096;
      * the skinny and batched GEMMs;
      * the 12-layer chain at 4096 tokens (the linear step, forward and
        backward of 48 linears, graph-replayed) against the roofline of its
        GEMM FLOPs and quantize bytes."""
    import torch
    dev = torch.device("cuda:0")
    gen = torch.Generator("cuda").manual_seed(7)
    codes = lambda *shape: torch.randint(0, 120, shape, dtype=torch.uint8, device=dev, generator=gen)
    s_a, s_b = torch.tensor([0.0123], device=dev), torch.tensor([0.0217], device=dev)

    def gemm(name, layout, m, n, k, batch=1, bcast=False, bias=False, fa=0):
        a_shape = (k, m) if layout == ds.TN else (m, k)
        b_shape = (n, k) if layout == ds.NT else (k, n)
        per = batch * m * k + (1 if bcast else batch) * n * k + 2 * batch * m * n + (2 * n if bias else 0)
        rot = max(1, min(64, -(-(512 << 20) // per)))
        A = [codes(batch, *a_shape) for _ in range(rot)]
        B = [codes(1 if bcast else batch, *b_shape) for _ in range(rot)]
        C = [torch.empty((batch, m, n), dtype=torch.bfloat16, device=dev) for _ in range(rot)]
        bv = torch.randn(n, device=dev, generator=gen).to(torch.bfloat16) if bias else None
        kw = dict(batch=batch, stride_a=m * k, stride_b=0 if bcast else n * k, stride_c=m * n) if batch > 1 else {}
        fn = lambda i: ds.fp8_mm(A[i % rot], B[i % rot], fa, ds.E4M3, layout, m, n, k, s_a, s_b, bias=bv,
                                 out=C[i % rot], **kw)
        ms = time_each(fn, stream, reps=60 if 2.0 * m * n * k * batch > 1e11 else 100, warmup=20)
        lay = {ds.NT: "NT", ds.NN: "NN", ds.TN: "TN"}[layout]
        desc = (f"{'bmm ' + str(batch) + ' x ' if batch > 1 else ''}{m}x{n}x{k} {lay}"
                f"{' B broadcast' if bcast else ''}{' + bf16 bias' if bias else ''}"
                f" {'E5M2' if fa else 'E4M3'} x E4M3, bf16 out, inputs rotated over {rot} copies")
        return gemm_entry(ms, m, n, k, batch, per, desc)

    def quant(name, rows, cols, fmt, sigma):
        n = rows * cols
        rot = max(1, min(64, -(-(512 << 20) // (3 * n))))
        X = [(torch.randn(rows, cols, device=dev, generator=gen) * sigma).to(torch.bfloat16) for _ in range(rot)]
        Y = [torch.empty((rows, cols), dtype=torch.uint8, device=dev) for _ in range(rot)]
        ring = ds.ScaleRing(16, fmt)
        ms = time_each(lambda i: ds.fp8_quantize(X[i % rot], fmt, ring, out=Y[i % rot]), stream, reps=100,
                       warmup=20)
        us = spread_us(ms)["p50"]
        gbps = 3.0 * n / (us * 1e-6) / 1e9
        return {"workload": f"{rows}x{cols} bf16 -> {'E5M2' if fmt else 'E4M3'}, history 16, "
                            f"inputs rotated over {rot} copies",
                "us_p50": us, "launch_us": spread_us(ms), "gbps": round(gbps, 1), "bound": "hbm",
                "frac": round(gbps / PEAK_HBM_GBPS, 4), "roofline_us": round(3.0 * n / PEAK_HBM_GBPS / 1e3, 2),
                "bytes": 3.0 * n}

    def linear_layer():
        return {
            "gemm_fwd_nt": gemm("fwd", ds.NT, 2048, 4096, 1024, bias=True),
            "gemm_dx_nn": gemm("dx", ds.NN, 2048, 1024, 4096, fa=1),
            "gemm_dw_tn": gemm("dw", ds.TN, 4096, 1024, 2048, fa=1),
            "quantize_x": quant("x", 2048, 1024, ds.E4M3, 1.0),
            "quantize_w": quant("w", 4096, 1024, ds.E4M3, 1.0),
            "quantize_g": quant("g", 2048, 4096, ds.E5M2, 1e-3),
        }

    def skinny_batched():
        return {
            "64x8192x2048": gemm("s1", ds.NT, 64, 8192, 2048),
            "1024x1536x2048": gemm("s2", ds.NT, 1024, 1536, 2048),
            "1024x1000x2048_bias": gemm("s3", ds.NT, 1024, 1000, 2048, bias=True),
            "bmm_64x512x512x512": gemm("s4", ds.NT, 512, 512, 512, batch=64),
            "bmm_8x1024x1024x2048_b_broadcast": gemm("s5", ds.NT, 1024, 1024, 2048, batch=8, bcast=True),
        }

    def chain():
        c = measure_linear_step(stream, tokens=4096)
        # Roofline of the chain: its GEMM FLOPs at the MFMA peak plus the bytes
        # of its 144 quantizes (2 B read + 1 B written per element) at HBM peak.
        dims = [(1024, 3072), (1024, 1024), (1024, 4096), (4096, 1024)] * 12
        q_bytes = 3.0 * sum(4096 * i + o * i + 4096 * o for i, o in dims)
        roof_ms = c["gemm_flops"] / (PEAK_FP8_TFLOPS * 1e12) * 1e3 + q_bytes / (PEAK_HBM_GBPS * 1e9) * 1e3
        c["roofline_ms"] = round(roof_ms, 3)
        c["frac"] = round(roof_ms / c["fp8_ms_per_step"], 4)
        return c

    out = {}
    want = lambda name: only is None or only == name
    if want("linear_d1024_t2048"):
        out["linear_d1024_t2048"] = linear_layer()
    if want("square_sweep"):
        torch.cuda.empty_cache()
        out["square_sweep"] = {str(n): gemm(f"sq{n}", ds.NT, n, n, n) for n in (1024, 2048, 4096)}
    if want("skinny_batched"):
        torch.cuda.empty_cache()
        out["skinny_batched"] = skinny_batched()
    if want("chain_12_layers_t4096"):
        torch.cuda.empty_cache()
        out["chain_12_layers_t4096"] = chain()
    return out


def measure_linear_overhead(stream, reps=200):
    """Fixed cost of one FP8 linear layer: forward + backward of a layer whose
    arithmetic is negligible (16 tokens, 128 -> 128, with bias), per call,
    eagerly (host work + the launches: a batched quantize of X and W, the NT
    GEMM, the quantize of G, the dX + dW pair and the bias gradient) and
    replayed from a HIP graph (device time of that launch chain only); the
    same for torch's bf16 linear."""
    import torch
    from delayed_scaling_amd.linear import Fp8Linear
    x = torch.randn(16, 128, device="cuda").to(torch.bfloat16).requires_grad_()
    g = torch.randn(16, 128, device="cuda").to(torch.bfloat16)
    mods = {"fp8": Fp8Linear(128, 128, bias=True),
            "bf16": torch.nn.Linear(128, 128, bias=True, device="cuda", dtype=torch.bfloat16)}
    res = {}
    for name, mod in mods.items():
        def run():
            x.grad = None
            for prm in mod.parameters():
                prm.grad = None
            mod(x).backward(g)
        for _ in range(20):
            run()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            run()
        torch.cuda.synchronize()
        res[name + "_eager_us"] = round((time.perf_counter() - t0) / reps * 1e6, 2)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run()
        ms = time_each(lambda i: graph.replay(), stream, reps=reps, warmup=10)
        res[name + "_graph_us"] = spread_us(ms)["p50"]
    res["workload"] = ("forward + backward of one linear layer, 16 tokens, 128 -> 128 with bias (the fixed "
                       "cost per linear); eager: host time per call with the launches; graph: replay time")
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import delayed_scaling_amd as ds
    from synth import bf16_normal, seed_for

    n = args.size
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.only_config:
        # One group of the per-config workloads and nothing else (to profile it).
        print(json.dumps({"configs": measure_configs(ds, stream, only=args.only_config)}), flush=True)
        return

    a_bits = bf16_normal((n, n), seed_for(3, 0, "A"))
    b_bits = bf16_normal((n, n), seed_for(3, 0, "B"))
    to_dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    a0, b0 = to_dev(a_bits), to_dev(b_bits)
    rot = max(1, args.rotate)
    A = [a0] + [a0.clone() for _ in range(rot - 1)]
    B = [b0] + [b0.clone() for _ in range(rot - 1)]
    A8 = [torch.empty((n, n), dtype=torch.uint8, device=dev) for _ in range(rot)]
    B8 = [torch.empty((n, n), dtype=torch.uint8, device=dev) for _ in range(rot)]
    C = [torch.empty((n, n), dtype=torch.bfloat16, device=dev) for _ in range(rot)]
    ring_a = ds.ScaleRing(16, ds.E4M3)
    ring_b = ds.ScaleRing(16, ds.E4M3)

    # Calibration copy of known size for the HBM counters (a device-to-device
    # copy of 256 MiB, read once and written once).
    cal_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)

    def step(i, ev=None):
        r = i % rot
        if ev is not None:
            ev[0].record(stream)
        # A and B in one launch, each with its own ring.
        ds.fp8_quantize_batch([A[r], B[r]], ds.E4M3, [ring_a, ring_b], outs=[A8[r], B8[r]])
        if ev is not None:
            ev[1].record(stream)
        ds.fp8_mm(A8[r], B8[r], ds.E4M3, ds.E4M3, ds.NT, n, n, n, ring_a, ring_b, out=C[r])
        if ev is not None:
            ev[2].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Untimed steps until --settle-ms have passed: the shader clock ramps for
    # tens of milliseconds once this load starts.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step(args.warmup + settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    first = args.warmup + settle_steps

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(first + i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_step = (t1 - t0) * 1e3 / args.steps
    q_ms = [e[0].elapsed_time(e[1]) for e in events]
    g_ms = [e[1].elapsed_time(e[2]) for e in events]

    def spread(ms):
        """p10 / median / p90 of per-step launch times, in microseconds."""
        v = sorted(ms)
        pick = lambda f: round(v[min(len(v) - 1, int(f * len(v)))] * 1e3, 2)
        return {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9)}
    q_avg = sum(q_ms) / len(q_ms)
    g_avg = sum(g_ms) / len(g_ms)
    flops = 2.0 * n * n * n
    q_bytes = 6.0 * n * n       # two n x n bf16 tensors read, their codes written

    def quantize_after(pred, reps=30):
        """Median duration (us) of the step's quantize launch issued right
        after pred(r) on the same stream (None: after the device went idle);
        events bracket the quantize alone."""
        evs = []
        for i in range(reps):
            r = i % rot
            if pred is None:
                torch.cuda.synchronize()
            else:
                pred(r)
            e = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            e[0].record(stream)
            ds.fp8_quantize_batch([A[r], B[r]], ds.E4M3, [ring_a, ring_b], outs=[A8[r], B8[r]])
            e[1].record(stream)
            evs.append(e)
        torch.cuda.synchronize()
        return spread([a.elapsed_time(b) for a, b in evs])["p50"]

    q_after = {
        "gemm": quantize_after(lambda r: ds.fp8_mm(A8[r], B8[r], ds.E4M3, ds.E4M3, ds.NT, n, n, n, ring_a, ring_b,
                                                   out=C[r])),
        "copy_256MiB": quantize_after(lambda r: cal_dst.copy_(cal_src)),
        "quantize": quantize_after(lambda r: ds.fp8_quantize_batch([A[r], B[r]], ds.E4M3, [ring_a, ring_b],
                                                                   outs=[A8[r], B8[r]])),
        "idle": quantize_after(None),
    }
    q_after = {k: {"p50_us": v, "frac": round(q_bytes / (v * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
               for k, v in q_after.items()}
    q_after["note"] = ("the same quantize launch after different predecessors: the step's GEMM, a streaming "
                       "device copy, itself, or an idle device")
    gemm_tflops = flops / (g_avg * 1e-3) / 1e12
    q_gbps = q_bytes / (q_avg * 1e-3) / 1e9
    traffic = traffic_from_profile(GEMM_SOURCES, "kernel_source_sha256", "hbm_bytes_per_launch")
    q_traffic = traffic_from_profile(QUANT_SOURCES, "quantize_source_sha256", "quantize_batch_hbm_bytes_per_launch")

    out = {
        "metric": "FP8 GEMM TFLOP/s (E4M3 NT 8192^3) + quantize GB/s, % of MI355X peak",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 (fp32 accumulate, bf16 out)",
        "data": "synthetic",
        "config": {"workload": f"square E4M3 NT {n}^3: delayed-scaling quantize of A and B ({n}x{n} bf16 "
                               f"~N(0,1), history 16) + scaled FP8 GEMM, bf16 out, no bias",
                   "m": n, "n": n, "k": n, "hist_len": 16, "input_rotation": rot},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "gemm_u128_kernel<NT, E4M3 x E4M3>: 256x256 tile, 4 waves, 128-byte K units",
                     "avg_launch_us": round(g_avg * 1e3, 2), "launch_us": spread(g_ms)},
        "clock_settle": {"ms": round(settle_ms, 1), "steps": settle_steps,
                         "note": "untimed steps after the warm-up steps, before the timed ones"},
        "roofline_quantize": {"bound": "hbm", "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS,
                              "unit": "GB/s", "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
                              "traffic": q_traffic,
                              "kernel": "quantize_batch_kernel<E4M3>: A and B, each with its ring, one launch",
                              "bytes_per_launch": q_bytes,
                              "avg_launch_us": round(q_avg * 1e3, 2), "launch_us": spread(q_ms),
                              "after_predecessor": q_after},
    }
    if not args.no_widened:
        del A, B, A8, B8, C, cal_src, cal_dst
        torch.cuda.empty_cache()
        out["widened"] = measure_widened(ds, n, stream)
        if not args.no_linear_step:
            out["widened"]["linear_step_12_layers"] = measure_linear_step(stream)
        qsrc, gsrc = QUANT_SOURCES, GEMM_SOURCES
        for name, entry in out["widened"].items():
            if "bound" not in entry:
                continue
            src, sha_key = (gsrc, "kernel_source_sha256") if name.startswith("gemm") else (qsrc, "quantize_source_sha256")
            key = {"gemm_nn_dx": "gemm_nn", "gemm_tn_dw": "gemm_tn"}.get(name, name) + "_hbm_bytes_per_launch"
            if name == "quantize_dynamic":
                a = traffic_from_profile(qsrc, sha_key, "amax_hbm_bytes_per_launch")
                q = traffic_from_profile(qsrc, sha_key, "quantize_single_hbm_bytes_per_launch")
                entry["traffic"] = None if a is None or q is None else a + q
            else:
                entry["traffic"] = traffic_from_profile(src, sha_key, key)
    if not args.no_configs:
        out["configs"] = measure_configs(ds, stream)
        out["per_linear_overhead"] = measure_linear_overhead(stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a_bits, b_bits, n, min(args.cpu_rows, n))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
