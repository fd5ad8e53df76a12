"""Parity of the batched quantize (several tensors, each with its own ring, in
one launch) with the oracle's quantize step applied to each tensor on its own,
and of the ring update for history windows longer than one wavefront.  Codes,
ring fields and the applied 1/scale written for the caller are bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import f32_bits, require_gpu, say, to_dev_bf16
from synth import bf16_from_float, bf16_normal
from test_gpu_quantize import assert_ring_equal
from test_gpu_widen import make_input, to_dev

pytestmark = pytest.mark.gpu

def check_batch(ds, xs_bits, kind, fmt, rings, refs, with_scale_out=True):
    """One batched call on both sides; returns the advanced oracle rings."""
    n = len(xs_bits)
    s = torch.full((n,), -1.0, dtype=torch.float32, device="cuda")
    outs = ds.fp8_quantize_batch([to_dev(x, kind) for x in xs_bits], fmt, rings,
                                 scale_inv_outs=[s[i:i + 1] for i in range(n)] if with_scale_out else None)
    torch.cuda.synchronize()
    s_host = s.cpu().numpy()
    new = []
    for i, x in enumerate(xs_bits):
        codes, r = oracle.quantize_step(refs[i], x, kind)
        assert np.array_equal(outs[i].cpu().numpy(), codes), i
        assert_ring_equal(rings[i].read(), r, i)
        if with_scale_out and x.size:
            assert f32_bits(s_host[i]) == f32_bits(r.scale_inv_used), i
        new.append(r)
    return new


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_batch_matches_oracle_per_job(fmt):
    """Ragged sizes (a linear's X and W, a tail shorter than one 16-byte chunk,
    a tensor smaller than one chunk), three steps with the amax changing."""
    ds = require_gpu()
    sizes = [2048 * 1024, 1024 * 4096 + 8, 100003, 5, 16]
    rings = [ds.ScaleRing(16, fmt) for _ in sizes]
    refs = [oracle.ring_init(16, fmt) for _ in sizes]
    for step in range(3):
        say(f"batch fmt={fmt} step {step}")
        xs = [bf16_normal((n,), 700 + 10 * step + i, 2.0 ** (2 * step - 2) * (i + 1), outliers=True)
              for i, n in enumerate(sizes)]
        refs = check_batch(ds, xs, oracle.IN_BF16, fmt, rings, refs)


@pytest.mark.parametrize("kind", [oracle.IN_F16, oracle.IN_F32])
def test_batch_input_types_equal_single_calls(kind):
    """The batch gives the bytes of one fp8_quantize call per tensor, and the
    same ring bytes, step after step."""
    ds = require_gpu()
    sizes = [300001, 65536, 3]
    rb = [ds.ScaleRing(4, oracle.E5M2, 2.0) for _ in sizes]
    rs = [ds.ScaleRing(4, oracle.E5M2, 2.0) for _ in sizes]
    refs = [oracle.ring_init(4, oracle.E5M2, 2.0) for _ in sizes]
    for step in range(3):
        say(f"batch kind={kind} step {step}")
        xs = [make_input((n,), 800 + 10 * step + i, kind, sigma=4.0 * (step + 1)) for i, n in enumerate(sizes)]
        single = [ds.fp8_quantize(to_dev(x, kind), oracle.E5M2, r) for x, r in zip(xs, rs)]
        outs = ds.fp8_quantize_batch([to_dev(x, kind) for x in xs], oracle.E5M2, rb)
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            codes, refs[i] = oracle.quantize_step(refs[i], x, kind)
            assert np.array_equal(outs[i].cpu().numpy(), codes), i
            assert torch.equal(single[i], outs[i]), i
            assert rs[i].read() == rb[i].read(), i
            assert_ring_equal(rb[i].read(), refs[i], i)


def test_batch_of_eight_with_empty_jobs():
    """The largest batch; empty jobs leave their rings untouched and take no
    blocks; no scale_inv outputs requested."""
    ds = require_gpu()
    sizes = [0, 4096, 0, 1 << 20, 7, 0, 123457, 64]
    rings = [ds.ScaleRing(3, oracle.E4M3, 0.5) for _ in sizes]
    refs = [oracle.ring_init(3, oracle.E4M3, 0.5) for _ in sizes]
    for step in range(2):
        say(f"batch of eight step {step}")
        xs = [bf16_normal((n,), 900 + 10 * step + i, 3.0) for i, n in enumerate(sizes)]
        before = [r.read() for r in rings]
        outs = ds.fp8_quantize_batch([to_dev_bf16(x) for x in xs], oracle.E4M3, rings)
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            if x.size == 0:
                assert rings[i].read() == before[i], i
                continue
            codes, refs[i] = oracle.quantize_step(refs[i], x)
            assert np.array_equal(outs[i].cpu().numpy(), codes), i
            assert_ring_equal(rings[i].read(), refs[i], i)


def test_batch_interleaved_with_single_calls_on_one_ring():
    """A ring used by single calls and by batches in turn stays one ring."""
    ds = require_gpu()
    ring, other = ds.ScaleRing(5, oracle.E4M3), ds.ScaleRing(5, oracle.E4M3)
    ref, ref_o = oracle.ring_init(5, oracle.E4M3), oracle.ring_init(5, oracle.E4M3)
    for step in range(6):
        x = bf16_normal((70000,), 950 + step, 2.0 ** (step % 3), outliers=True)
        if step % 2:
            q = ds.fp8_quantize(to_dev_bf16(x), oracle.E4M3, ring)
            codes, ref = oracle.quantize_step(ref, x)
            torch.cuda.synchronize()
            assert np.array_equal(q.cpu().numpy(), codes), step
            assert_ring_equal(ring.read(), ref, step)
        else:
            y = bf16_normal((333,), 960 + step, 1.0)
            ref, ref_o = check_batch(ds, [x, y], oracle.IN_BF16, oracle.E4M3, [ring, other], [ref, ref_o])


@pytest.mark.parametrize("hist_len", [1, 63, 64, 65, 130, 1024])
def test_long_history_windows(hist_len):
    """Windows beyond the 64 entries read at launch: a spike in the amax at
    step 1 holds the scale down for exactly hist_len steps, then leaves the
    window (for the 1024-entry window, 70 steps fill entries past 64)."""
    ds = require_gpu()
    steps = hist_len + 3 if hist_len <= 130 else 70
    ring = ds.ScaleRing(hist_len, oracle.E4M3)
    ref = oracle.ring_init(hist_len, oracle.E4M3)
    base = bf16_normal((4097,), 990, 1.0)
    base_f = (base.astype(np.uint32) << 16).view(np.float32)
    say(f"history {hist_len}: {steps} steps")
    for t in range(steps):
        f = 64.0 if t == 1 else 1.0 + 0.125 * (t % 5)
        x = bf16_from_float(base_f * np.float32(f))
        q = ds.fp8_quantize(to_dev_bf16(x), oracle.E4M3, ring)
        codes, ref = oracle.quantize_step(ref, x)
        if t % 7 == 0 or t >= steps - 3 or t <= 2 or t in (hist_len, hist_len + 1):
            torch.cuda.synchronize()
            assert np.array_equal(q.cpu().numpy(), codes), t
            assert_ring_equal(ring.read(), ref, t)
    torch.cuda.synchronize()
    assert_ring_equal(ring.read(), ref, "end")


def test_batch_at_the_bench_step_configuration():
    """A and B of the headline workload (8192 x 8192 bf16 each, history 16) in
    one batched launch, as the benchmark step issues them: two steps, codes,
    rings and applied 1/scale outputs bit-exact against the oracle."""
    ds = require_gpu()
    from synth import seed_for
    a = bf16_normal((8192, 8192), seed_for(3, 0, "A"))
    b = bf16_normal((8192, 8192), seed_for(3, 0, "B"))
    rings = [ds.ScaleRing(16, oracle.E4M3), ds.ScaleRing(16, oracle.E4M3)]
    refs = [oracle.ring_init(16, oracle.E4M3), oracle.ring_init(16, oracle.E4M3)]
    for step in range(2):
        say(f"bench-configuration batch step {step}")
        refs = check_batch(ds, [a.reshape(-1), b.reshape(-1)], oracle.IN_BF16, oracle.E4M3, rings, refs)
