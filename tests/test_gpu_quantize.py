"""Parity of the HIP quantize + scale-ring kernel with the oracle: codes and
every ring field bit-exact, on every bf16 pattern, the tiny doubling
workload, a multi-step outlier chain, ragged sizes, the full 8192 x 8192
operand, NaN / inf, empty inputs, format mismatch, checkpoint / restore."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, f32_bits, require_gpu, say, to_dev_bf16
from synth import all_bf16_patterns, bf16_from_float, bf16_normal, seed_for

pytestmark = pytest.mark.gpu


def assert_ring_equal(gpu, ref, where=""):
    assert gpu["scale_bits"] == f32_bits(ref.scale), (where, gpu["scale"], ref.scale)
    assert gpu["scale_inv_used_bits"] == f32_bits(ref.scale_inv_used), (where, gpu["scale_inv_used"], ref.scale_inv_used)
    assert gpu["amax_last_bits"] == f32_bits(ref.amax_last), where
    assert gpu["idx"] == ref.idx, where
    assert gpu["hist_bits"] == [int(v) for v in ref.hist.view(np.uint32)], where
    assert gpu["amax_bits"] == 0 and gpu["ticket"] == 0 and gpu["status"] == 0, where
    assert gpu["group_scratch_zero"], where


def run_steps(ds, xs, fmt, hist_len, init_scale=1.0):
    """Quantize a sequence of tensors through one ring on both sides."""
    ring = ds.ScaleRing(hist_len, fmt, init_scale)
    ref = oracle.ring_init(hist_len, fmt, init_scale)
    for t, x in enumerate(xs):
        q = ds.fp8_quantize(to_dev_bf16(x), fmt, ring)
        codes, ref = oracle.quantize_step(ref, x)
        torch.cuda.synchronize()
        got = q.cpu().numpy()
        assert np.array_equal(got, codes), (t, np.flatnonzero(got != codes)[:10])
        assert_ring_equal(ring.read(), ref, f"step {t}")
    return ring, ref


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_every_bf16_pattern_and_scale(fmt):
    ds = require_gpu()
    x = all_bf16_patterns()
    for scale in [1.0, 448.0 / 3.25, 2.0 ** -20, 2.0 ** 20, 57344.0 / 7.0, 1.0 / 3.0, 1e-30, 3e30]:
        say(f"every pattern fmt={fmt} scale={scale}")
        ring = ds.ScaleRing(4, fmt, scale)
        q = ds.fp8_quantize(to_dev_bf16(x), fmt, ring)
        ref = oracle.ring_init(4, fmt, scale)
        codes, ref = oracle.quantize_step(ref, x)
        torch.cuda.synchronize()
        got = q.cpu().numpy()
        bad = np.flatnonzero(got != codes)
        assert bad.size == 0, [(hex(int(x[i])), hex(int(got[i])), hex(int(codes[i]))) for i in bad[:8]]
        assert_ring_equal(ring.read(), ref)


def test_tiny_doubling_workload():
    """64 x 64 X and W, history 4, three steps with the amax doubling."""
    ds = require_gpu()
    for tensor in ("X", "W"):
        x0 = bf16_normal((64, 64), 0 if tensor == "X" else seed_for(1, 0, "W"))
        xs = []
        for t in range(3):
            xt = (oracle.bf16_to_f32(x0) * np.float32(2.0 ** t)).astype(np.float32)
            xs.append((xt.view(np.uint32) >> 16).astype(np.uint16))
        run_steps(ds, xs, oracle.E4M3, 4)


@pytest.mark.parametrize("fmt,sigma", [(oracle.E4M3, 1.0), (oracle.E5M2, 1e-3)])
def test_outlier_chain_sixteen_history(fmt, sigma):
    """History 16, 20 steps (wraps), 1% outliers x50, changing sizes."""
    ds = require_gpu()
    sizes = [4096 * 1024, 1000, 777777, 65536, 8, 3]
    xs = [bf16_normal((sizes[t % len(sizes)],), seed_for(5, t, "G"), sigma * (1 + t % 4), outliers=True)
          for t in range(20)]
    run_steps(ds, xs, fmt, 16)


@pytest.mark.parametrize("numel", [1, 7, 8, 9, 15, 1023, 4097, 262144 + 5, 1048576 * 3 + 1])
def test_ragged_sizes(numel):
    ds = require_gpu()
    x = bf16_normal((numel,), 1234 + numel, 3.0)
    run_steps(ds, [x, x[::-1].copy()], oracle.E4M3, 2)


def test_full_size_operand_8192_squared():
    """The 8192 x 8192 bf16 operand (the largest grid: every block takes a
    ticket), two steps, bit-exact."""
    ds = require_gpu()
    x = bf16_normal((8192, 8192), seed_for(3, 0, "A"))
    say("full-size quantize 8192^2")
    run_steps(ds, [x, x], oracle.E4M3, 16)


def test_nan_inf_and_huge_inputs():
    ds = require_gpu()
    base = bf16_normal((5000,), 77, 10.0)
    x = base.copy()
    x[[3, 100, 4096]] = [0x7FC0, 0xFFC1, 0x7F81]       # NaNs of both signs
    x[[5, 6]] = [0x7F80, 0xFF80]                        # +-inf
    x[7] = 0x7F7F                                       # largest finite bf16
    y = base.copy()
    y[[11, 12]] = [0x7F80, 0xFF80]
    run_steps(ds, [base, x, y, base], oracle.E4M3, 3)
    run_steps(ds, [base, x, y, base], oracle.E5M2, 3)


def test_empty_input_leaves_ring_unchanged():
    ds = require_gpu()
    ring = ds.ScaleRing(4, oracle.E4M3, 2.0)
    before = ring.read()
    q = ds.fp8_quantize(torch.empty(0, dtype=torch.bfloat16, device="cuda"), oracle.E4M3, ring)
    torch.cuda.synchronize()
    assert q.numel() == 0 and ring.read() == before


def test_format_mismatch_sets_status_and_keeps_state():
    ds = require_gpu()
    ring = ds.ScaleRing(4, oracle.E4M3, 1.0)
    x = to_dev_bf16(bf16_normal((1000,), 5))
    ds.fp8_quantize(x, oracle.E4M3, ring)
    before = ring.read()
    ds.fp8_quantize(x, oracle.E5M2, ring)
    after = ring.read()
    assert after["status"] == 1
    for key in ("scale_bits", "scale_inv_used_bits", "idx", "hist_bits", "amax_last_bits"):
        assert after[key] == before[key]
    assert after["amax_bits"] == 0 and after["ticket"] == 0


def test_checkpoint_restore_continues_identically():
    ds = require_gpu()
    xs = [bf16_normal((100000,), 900 + t, 1.0 + t, outliers=True) for t in range(6)]
    ring = ds.ScaleRing(4, oracle.E4M3)
    for x in xs[:3]:
        ds.fp8_quantize(to_dev_bf16(x), oracle.E4M3, ring)
    saved = ring.buf.clone()
    out1 = [ds.fp8_quantize(to_dev_bf16(x), oracle.E4M3, ring).cpu() for x in xs[3:]]
    end1 = ring.read()
    ring.buf.copy_(saved)
    out2 = [ds.fp8_quantize(to_dev_bf16(x), oracle.E4M3, ring).cpu() for x in xs[3:]]
    assert ring.read() == end1
    assert all(torch.equal(a, b) for a, b in zip(out1, out2))
