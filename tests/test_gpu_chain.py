"""The training-chain workload: tokens 4096, model dim 1024, the four linears
of one transformer layer (QKV 1024->3072, O 1024->1024, MLP up 1024->4096,
down 4096->1024) for 10 steps, history 16, fresh inputs every step with 1%
outliers x50 on X, W and G; forward E4M3, backward E5M2, the scales each step
publishes used by the next.  The twelve rings are compared with the oracle
bit for bit after every call.  Each step one linear (in turn) also has its
quantized bytes compared in full and its three GEMMs on sampled entries.

The second test runs the workload at its stated size: twelve layers (144
rings) for 10 steps, inputs drawn on the GPU (bf16_normal_device) so the
step's 0.9 G elements need not be drawn on the host; every ring is compared
with the oracle bit for bit after every call, and each step one linear in
turn (spread over the layers) has its codes compared in full and its three
GEMMs on the first and last row and column of every 256 x 256 output tile."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import require_gpu, say, to_dev_bf16
from synth import bf16_normal, bf16_normal_device, seed_for
from test_gpu_configs import Side, check_mm, check_mm_tiles

pytestmark = pytest.mark.gpu
E4M3, E5M2 = oracle.E4M3, oracle.E5M2
TOKENS = 4096
LINEARS = [("qkv", 1024, 3072), ("o", 1024, 1024), ("up", 1024, 4096), ("down", 4096, 1024)]


def test_one_layer_ten_steps():
    ds = require_gpu()
    rings = {name: (Side(ds, E4M3, 16), Side(ds, E4M3, 16), Side(ds, E5M2, 16)) for name, _, _ in LINEARS}
    for step in range(10):
        for li, (name, din, dout) in enumerate(LINEARS):
            full = li == step % len(LINEARS)
            say(f"chain step {step} {name} full={full}")
            x = bf16_normal((TOKENS, din), seed_for(5, step, "X", li), 1.0, outliers=True)
            w = bf16_normal((dout, din), seed_for(5, step, "W", li), 1.0, outliers=True)
            g = bf16_normal((TOKENS, dout), seed_for(5, step, "G", li), 1e-3, outliers=True)
            sx, sw, sg = rings[name]
            qx, cx = sx.quantize(x, check_codes=full)
            qw, cw = sw.quantize(w, check_codes=full)
            y = ds.fp8_mm(qx, qw, E4M3, E4M3, ds.NT, TOKENS, dout, din, sx.ring, sw.ring)
            qg, cg = sg.quantize(g, check_codes=full)
            dx = ds.fp8_mm(qg, qw, E5M2, E4M3, ds.NN, TOKENS, din, dout, sg.ring, sw.ring)
            dw = ds.fp8_mm(qg, qx, E5M2, E4M3, ds.TN, dout, din, TOKENS, sg.ring, sx.ring)
            if full:
                check_mm(ds, y, cx, cw, E4M3, E4M3, oracle.NT, TOKENS, dout, din, sx.s_inv, sw.s_inv,
                         sample=1500, what=f"{name} fwd step {step}")
                check_mm(ds, dx, cg, cw, E5M2, E4M3, oracle.NN, TOKENS, din, dout, sg.s_inv, sw.s_inv,
                         sample=1500, what=f"{name} dX step {step}")
                check_mm(ds, dw, cg, cx, E5M2, E4M3, oracle.TN, dout, din, TOKENS, sg.s_inv, sx.s_inv,
                         sample=1500, what=f"{name} dW step {step}")
    # after ten steps every ring has published scales from a full window
    for name, _, _ in LINEARS:
        for side in rings[name]:
            assert side.ref.idx == 10 % 16


def test_twelve_layers_ten_steps():
    ds = require_gpu()
    layers = 12
    rings = {(layer, name): (Side(ds, E4M3, 16), Side(ds, E4M3, 16), Side(ds, E5M2, 16))
             for layer in range(layers) for name, _, _ in LINEARS}
    for step in range(10):
        full_at = (step * 13) % (layers * len(LINEARS))
        say(f"12-layer chain step {step}, full check of linear {full_at}")
        for layer in range(layers):
            for li, (name, din, dout) in enumerate(LINEARS):
                idx = layer * len(LINEARS) + li
                full = idx == full_at
                x = bf16_normal_device((TOKENS, din), seed_for(6, step, "X", idx), 1.0, outliers=True)
                w = bf16_normal_device((dout, din), seed_for(6, step, "W", idx), 1.0, outliers=True)
                g = bf16_normal_device((TOKENS, dout), seed_for(6, step, "G", idx), 1e-3, outliers=True)
                sx, sw, sg = rings[(layer, name)]
                qx, cx = sx.quantize(x, check_codes=full)
                qw, cw = sw.quantize(w, check_codes=full)
                y = ds.fp8_mm(qx, qw, E4M3, E4M3, ds.NT, TOKENS, dout, din, sx.ring, sw.ring)
                qg, cg = sg.quantize(g, check_codes=full)
                dx = ds.fp8_mm(qg, qw, E5M2, E4M3, ds.NN, TOKENS, din, dout, sg.ring, sw.ring)
                dw = ds.fp8_mm(qg, qx, E5M2, E4M3, ds.TN, dout, din, TOKENS, sg.ring, sx.ring)
                if full:
                    check_mm_tiles(ds, y, cx, cw, E4M3, E4M3, oracle.NT, TOKENS, dout, din, sx.s_inv, sw.s_inv,
                                   what=f"layer {layer} {name} fwd step {step}")
                    check_mm_tiles(ds, dx, cg, cw, E5M2, E4M3, oracle.NN, TOKENS, din, dout, sg.s_inv, sw.s_inv,
                                   what=f"layer {layer} {name} dX step {step}")
                    check_mm_tiles(ds, dw, cg, cx, E5M2, E4M3, oracle.TN, dout, din, TOKENS, sg.s_inv, sx.s_inv,
                                   what=f"layer {layer} {name} dW step {step}")
                del x, w, g, qx, qw, qg, y, dx, dw
    for side in (s for trio in rings.values() for s in trio):
        assert side.ref.idx == 10 % 16
