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
against HBM.  `cpu_baseline` times the oracle (numpy) on a bounded slice of
the same step on the host.
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
    # The clocks settle after about 75 steps (40 ms) of this workload; fewer
    # warm-up steps time part of the ramp.
    ap.add_argument("--warmup", type=int, default=150)
    ap.add_argument("--size", type=int, default=8192, help="M = N = K of the square workload")
    ap.add_argument("--rotate", type=int, default=3, help="input copies cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-rows", type=int, default=256, help="output rows of the oracle sample")
    ap.add_argument("--no-widened", action="store_true", help="skip the widened-path kernel timings")
    ap.add_argument("--no-linear-step", action="store_true", help="skip the 12-layer linear step")
    return ap.parse_args()


def traffic_from_profile(kernel_src, sha_key, bytes_key):
    """HBM bytes per launch recorded in profiles/ by the two PMC runs, or
    None when the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_8192_bench_kernels.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = hashlib.sha256(open(kernel_src, "rb").read()).hexdigest()
    m_sha = re.search(rf"^{sha_key}:\s*([0-9a-f]{{64}})", text, re.M)
    m_b = re.search(rf"^{bytes_key}:\s*([0-9.eE+]+)", text, re.M)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return float(m_b.group(1))


def cpu_baseline(a_bits, b_bits, size, rows):
    """The oracle as it stands on a bounded slice of the step: quantize all
    of B and the first `rows` rows of A, then the first `rows` output rows of
    the GEMM.  Scaled to the metric as GEMM FLOPs of the slice per second."""
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
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": (f"first {rows} of {size} output rows: quantize B ({size}x{size}) and {rows} rows of A, "
                       f"fp64 GEMM of the slice; {dt:.1f} s; numpy elementwise steps on 1 thread, "
                       f"the fp64 matmul on {blas_threads} BLAS threads")}


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
    2048 tokens (per layer QKV 1024->3072, O 1024->1024, MLP up 1024->4096 and
    down 4096->1024, no bias): the library's FP8 layer against torch's bf16
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
    for name, mods in (("fp8", fp8), ("bf16", bf16)):
        for _ in range(2):
            run(mods)
        res[name + "_eager"] = timed(lambda: run(mods))
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
            "eager_fp8_ms_per_step": round(res["fp8_eager"], 3), "eager_bf16_ms_per_step": round(res["bf16_eager"], 3)}


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

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
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
    gemm_tflops = flops / (g_avg * 1e-3) / 1e12
    q_gbps = q_bytes / (q_avg * 1e-3) / 1e9
    traffic = traffic_from_profile(os.path.join(ROOT, "delayed_scaling_amd", "csrc", "gemm.hip"),
                                   "kernel_source_sha256", "hbm_bytes_per_launch")
    q_traffic = traffic_from_profile(os.path.join(ROOT, "delayed_scaling_amd", "csrc", "quantize.hip"),
                                     "quantize_source_sha256", "quantize_batch_hbm_bytes_per_launch")

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
                     "traffic": traffic, "kernel": "gemm_kernel 256x256 tile, 4 waves, NT, E4M3 x E4M3",
                     "avg_launch_us": round(g_avg * 1e3, 2), "launch_us": spread(g_ms)},
        "roofline_quantize": {"bound": "hbm", "achieved": round(q_gbps, 1), "peak": PEAK_HBM_GBPS,
                              "unit": "GB/s", "frac": round(q_gbps / PEAK_HBM_GBPS, 4),
                              "traffic": q_traffic,
                              "kernel": "quantize_batch_kernel<E4M3>: A and B, each with its ring, one launch",
                              "bytes_per_launch": q_bytes,
                              "avg_launch_us": round(q_avg * 1e3, 2), "launch_us": spread(q_ms)},
    }
    if not args.no_widened:
        del A, B, A8, B8, C, cal_src, cal_dst
        torch.cuda.empty_cache()
        out["widened"] = measure_widened(ds, n, stream)
        if not args.no_linear_step:
            out["widened"]["linear_step_12_layers"] = measure_linear_step(stream)
        qsrc = os.path.join(ROOT, "delayed_scaling_amd", "csrc", "quantize.hip")
        gsrc = os.path.join(ROOT, "delayed_scaling_amd", "csrc", "gemm.hip")
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
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a_bits, b_bits, n, min(args.cpu_rows, n))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
