"""The widened kernels at the size the benchmark times them (8192 x 8192
operands, the benchmark's launch configuration), against the oracle: the
transposed and dual quantize, the dynamic recipe, fp16 / fp32 inputs (codes
bit-exact over the whole tensor, ring fields bit-exact), the bias gradient
(sampled columns within the float32 summation bound) and the backward GEMM
layouts at 8192^3 in E5M2 x E4M3 (sampled entries within the GEMM tolerance)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, require_gpu, say, to_dev_bf16, to_dev_u8
from synth import bf16_normal, random_codes, seed_for
from test_gpu_configs import check_mm, check_mm_tiles
from test_gpu_gemm import FINITE, scale_tensor
from test_gpu_quantize import assert_ring_equal
from test_gpu_widen import make_input, to_dev

pytestmark = pytest.mark.gpu

N = 8192


@pytest.mark.parametrize("layout", [oracle.TRANSPOSED, oracle.DUAL])
def test_orientations_at_full_size(layout):
    ds = require_gpu()
    x = bf16_normal((N, N), seed_for(3, 0, "X"), outliers=True)
    ring = ds.ScaleRing(16, oracle.E4M3)
    ref = oracle.ring_init(16, oracle.E4M3)
    for step in range(2):                       # the second step applies the published scale
        say(f"full-size orientation {layout} step {step}")
        y, y_t = ds.fp8_quantize_2d(to_dev_bf16(x), oracle.E4M3, ring, layout)
        codes = oracle.quantize_values(x, ref.scale, oracle.E4M3)
        ref = oracle.advance_ring(ref, oracle.amax(x))
        torch.cuda.synchronize()
        assert np.array_equal(y_t.cpu().numpy(), codes.T), step
        if layout == oracle.DUAL:
            assert np.array_equal(y.cpu().numpy(), codes), step
        assert_ring_equal(ring.read(), ref, step)


def test_dynamic_at_full_size():
    ds = require_gpu()
    x = bf16_normal((N, N), seed_for(3, 1, "X"), sigma=3.0, outliers=True)
    ring = ds.ScaleRing(1, oracle.E5M2)
    say("full-size dynamic")
    q = ds.fp8_quantize_dynamic(to_dev_bf16(x), oracle.E5M2, ring)
    a = oracle.amax(x)
    s = oracle.dynamic_scale(a, oracle.E5M2)
    codes = oracle.quantize_values(x, s, oracle.E5M2)
    ref = oracle.advance_ring(oracle.ring_init(1, oracle.E5M2, float(s)), a)   # a length-1 delayed ring
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), codes)
    assert_ring_equal(ring.read(), ref)


@pytest.mark.parametrize("kind", [oracle.IN_F16, oracle.IN_F32])
def test_input_types_at_full_size(kind):
    ds = require_gpu()
    x = make_input((N, N), 4000 + kind, kind, sigma=2.0)
    ring = ds.ScaleRing(16, oracle.E4M3, 3.0)
    ref = oracle.ring_init(16, oracle.E4M3, 3.0)
    say(f"full-size input type {kind}")
    q = ds.fp8_quantize(to_dev(x, kind), oracle.E4M3, ring)
    codes = oracle.quantize_values(x, ref.scale, oracle.E4M3, kind)
    ref = oracle.advance_ring(ref, oracle.amax(x, kind))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), codes)
    assert_ring_equal(ring.read(), ref)


def test_bias_grad_at_full_size():
    ds = require_gpu()
    g = bf16_normal((N, N), seed_for(3, 0, "G"), outliers=True)
    say("full-size bias gradient")
    ws = ds.BiasGradWorkspace(N, N)
    out = ds.fp8_bias_grad(to_dev_bf16(g), out_f32=True, workspace=ws)
    cols = np.sort(np.random.default_rng(8).choice(N, 128, replace=False))
    cols = np.concatenate([[0], cols, [N - 1]])
    sub = np.ascontiguousarray(g[:, cols])
    _, _, ref = oracle.bias_grad(sub, N, len(cols), oracle.IN_BF16)
    tol = oracle.bias_grad_tolerance(sub, N, len(cols), oracle.IN_BF16, ref, oracle.OUT_F32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()[cols].astype(np.float64)
    assert np.all(np.abs(got - ref.astype(np.float64)) <= tol)
    assert int(ws.buf.count_nonzero()) == 0                 # the workspace is clear again


@pytest.mark.parametrize("layout,fa", [(oracle.NT, oracle.E4M3), (oracle.NN, oracle.E5M2), (oracle.TN, oracle.E5M2)])
def test_layouts_at_full_size(layout, fa):
    """8192^3 in the forward (NT, E4M3 x E4M3) and backward (NN / TN, E5M2 x
    E4M3) formats: two whole rows and two whole columns of every 256 x 256
    output tile against the oracle."""
    ds = require_gpu()
    a = random_codes((N, N), 4100 + layout, FINITE[fa])
    b = random_codes((N, N), 4200 + layout, FINITE[oracle.E4M3])
    sa, sb = 0.0119, 0.0227
    say(f"full-size GEMM layout {layout}")
    y = ds.fp8_mm(to_dev_u8(a), to_dev_u8(b), fa, oracle.E4M3, layout, N, N, N, scale_tensor(sa),
                  scale_tensor(sb))
    torch.cuda.synchronize()
    check_mm_tiles(ds, y, a, b, fa, oracle.E4M3, layout, N, N, N, sa, sb, what=f"8192^3 layout {layout}")


def test_bias_gemm_at_full_size():
    """8192 x 8192 x 1024 NT with a bf16 bias: the automatic choice (the
    eight-wave 256x256 tile, bias staged through LDS) on sampled entries, and
    bit-equal to the four-wave tile's per-element bias path."""
    ds = require_gpu()
    m = n = N
    k = 1024
    a = random_codes((m, k), 4300, FINITE[oracle.E4M3])
    b = random_codes((n, k), 4301, FINITE[oracle.E4M3])
    bias = bf16_normal((n,), 4302)
    sa, sb = 0.0131, 0.0173
    say("full-size GEMM with bias")
    kw = dict(bias=to_dev_bf16(bias))
    y = ds.fp8_mm(to_dev_u8(a), to_dev_u8(b), oracle.E4M3, oracle.E4M3, oracle.NT, m, n, k, scale_tensor(sa),
                  scale_tensor(sb), **kw)
    y0 = ds.fp8_mm(to_dev_u8(a), to_dev_u8(b), oracle.E4M3, oracle.E4M3, oracle.NT, m, n, k, scale_tensor(sa),
                   scale_tensor(sb), tile=0, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y0.view(torch.int16))
    check_mm_tiles(ds, y, a, b, oracle.E4M3, oracle.E4M3, oracle.NT, m, n, k, sa, sb, bias=bias,
                   what="8192x8192x1024 NT with bias")
