"""The FP8 linear layer (autograd Function over the C ABI): it adds no
arithmetic of its own (outputs and gradients are the bits of the direct
library calls), its gradients follow the bf16 reference by direction and
norm, and it handles 3-D inputs, absent bias and masked gradients."""
import numpy as np
import pytest
import torch

from gpu_util import require_gpu, say
from synth import bf16_normal, seed_for

pytestmark = pytest.mark.gpu


def bf16(shape, seed, sigma=1.0, outliers=False):
    return torch.from_numpy(bf16_normal(shape, seed, sigma, outliers).view(np.int16)).view(torch.bfloat16).cuda()


def test_layer_equals_direct_calls():
    ds = require_gpu()
    from delayed_scaling_amd.linear import Fp8LinearState, fp8_linear
    t, n_in, n_out = 512, 256, 384
    x = bf16((t, n_in), seed_for(2, 0, "X")).requires_grad_()
    w = bf16((n_out, n_in), seed_for(2, 0, "W")).requires_grad_()
    b = bf16((n_out,), seed_for(2, 0, "bias")).requires_grad_()
    g = bf16((t, n_out), seed_for(2, 0, "G"), 1e-3)
    y = fp8_linear(x, w, b, Fp8LinearState(16))
    y.backward(g)
    # the same steps by hand on fresh rings
    rx, rw, rg = ds.ScaleRing(16, ds.E4M3), ds.ScaleRing(16, ds.E4M3), ds.ScaleRing(16, ds.E5M2)
    x8 = ds.fp8_quantize(x.detach(), ds.E4M3, rx)
    w8 = ds.fp8_quantize(w.detach(), ds.E4M3, rw)
    y_ref = ds.fp8_mm(x8, w8, ds.E4M3, ds.E4M3, ds.NT, t, n_out, n_in, rx, rw, bias=b.detach())
    g8 = ds.fp8_quantize(g, ds.E5M2, rg)
    dx = ds.fp8_mm(g8, w8, ds.E5M2, ds.E4M3, ds.NN, t, n_in, n_out, rg, rw)
    dw = ds.fp8_mm(g8, x8, ds.E5M2, ds.E4M3, ds.TN, n_out, n_in, t, rg, rx)
    db = ds.fp8_bias_grad(g)
    torch.cuda.synchronize()
    same = lambda p, q: torch.equal(p.reshape(-1).view(torch.int16), q.reshape(-1).view(torch.int16))
    assert same(y.detach(), y_ref) and same(x.grad, dx) and same(w.grad, dw) and same(b.grad, db)


def cos(a, b):
    a, b = a.float().reshape(-1), b.float().reshape(-1)
    return float((a @ b) / (a.norm() * b.norm()))


def test_gradients_follow_bf16_reference_over_steps():
    """Three training steps of a 3-D input [4, 512, 1024] through one layer;
    every step's output and gradients against float32 math on the same bf16
    values (direction > 0.99, norm within 3 %)."""
    require_gpu()
    from delayed_scaling_amd.linear import Fp8Linear
    layer = Fp8Linear(1024, 2048, bias=True)
    for step in range(3):
        say(f"linear step {step}")
        x = bf16((4, 512, 1024), seed_for(5, step, "X"), outliers=True).requires_grad_()
        g = bf16((4, 512, 2048), seed_for(5, step, "G"), 1e-3, outliers=True)
        layer.zero_grad()
        y = layer(x)
        y.backward(g)
        xf, wf, gf = x.detach().float(), layer.weight.detach().float(), g.float()
        y_ref = xf @ wf.t() + layer.bias.detach().float()
        dx_ref = gf @ wf
        dw_ref = gf.reshape(-1, 2048).t() @ xf.reshape(-1, 1024)
        db_ref = gf.reshape(-1, 2048).sum(0)
        for got, ref in [(y.detach(), y_ref), (x.grad, dx_ref), (layer.weight.grad, dw_ref), (layer.bias.grad, db_ref)]:
            assert cos(got, ref) > 0.99, step
            assert abs(float(got.float().norm() / ref.norm()) - 1) < 0.03, step
        with torch.no_grad():                         # a small update so the next step sees new weights
            layer.weight -= 1e-2 * layer.weight.grad.sign() * layer.weight.abs().mean()


def test_masks_and_no_bias():
    require_gpu()
    from delayed_scaling_amd.linear import Fp8Linear
    layer = Fp8Linear(256, 128, bias=False)
    x = bf16((64, 256), 3)                             # no grad for x
    y = layer(x)
    y.sum().backward()
    assert layer.weight.grad is not None and x.grad is None


def test_graph_replay_matches_eager():
    """A captured forward + backward of two layers replays to the bits of the
    eager run from the same ring state, three times, with eager work and
    synchronizations between the replays (no memset or host sync is captured)."""
    require_gpu()
    from delayed_scaling_amd.linear import Fp8Linear
    layers = [Fp8Linear(512, 768, bias=True), Fp8Linear(768, 512, bias=False)]
    x = bf16((256, 512), 41).requires_grad_()
    g = bf16((256, 512), 42, 1e-3)
    rings = [r for l in layers for r in (l.state.ring_x, l.state.ring_w, l.state.ring_g)]

    def step():
        y = layers[1](layers[0](x))
        y.backward(g)
        return y

    def reset(saved):
        for r, b in zip(rings, saved):
            r.buf.copy_(b)
        for p in [x] + [p for l in layers for p in l.parameters()]:
            if p.grad is not None:
                p.grad.zero_()

    saved = [r.buf.clone() for r in rings]
    y_eager = step().detach().clone()
    grads = [p.grad.clone() for p in [x] + [p for l in layers for p in l.parameters()]]
    rings_after = [r.buf.clone() for r in rings]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            reset(saved)
            step()
    torch.cuda.current_stream().wait_stream(s)
    reset(saved)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_static = step()
    for rep in range(3):
        reset(saved)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = lambda a, b: torch.equal(a.reshape(-1).view(torch.int16), b.reshape(-1).view(torch.int16))
        assert same(y_static, y_eager), rep
        for p, want in zip([x] + [p for l in layers for p in l.parameters()], grads):
            assert same(p.grad, want), rep
        for r, want in zip(rings, rings_after):
            assert torch.equal(r.buf, want), rep
        _ = (x.detach().float() * 2).sum().item()      # eager work between replays
