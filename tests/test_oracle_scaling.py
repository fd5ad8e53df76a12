"""Pins of oracle/scaling.py: amax against numpy's max, the quantize cast
against torch's float32 multiply + float8 cast over every bf16 pattern, and
the ring update against closed forms of workloads whose scales are known
exactly.  CPU only."""
import numpy as np
import pytest
import torch

from oracle import (E4M3, E5M2, FMAX, amax, bf16_to_f32, decode_fp8, quantize_step,
                    quantize_values, ring_init)
from synth import all_bf16_patterns, bf16_from_float, bf16_normal

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def f32_bits(x):
    return int(np.float32(x).view(np.uint32))


def test_amax_matches_numpy_max_abs():
    for seed, sigma in [(1, 1.0), (2, 1e-3), (3, 300.0)]:
        x = bf16_normal((257, 129), seed, sigma, outliers=True)
        ref = np.abs(bf16_to_f32(x)).max()
        assert f32_bits(amax(x)) == f32_bits(ref)


def test_amax_zero_sign_nan_inf():
    neg0 = np.array([0x8000, 0x8000], np.uint16)
    assert f32_bits(amax(neg0)) == 0
    x = bf16_from_float([1.0, -3.0, 2.0])
    assert amax(x) == np.float32(3.0)
    x_inf = bf16_from_float([1.0, -np.inf])
    assert amax(x_inf) == np.float32(np.inf)
    x_nan = np.concatenate([bf16_from_float([1.0, np.inf]), np.array([0xFFC1], np.uint16)])
    assert np.isnan(amax(x_nan))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_values_every_bf16_against_torch(fmt):
    x = all_bf16_patterns()
    xf = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
    finite = torch.isfinite(xf).numpy()
    for scale in [1.0, 448.0 / 3.25, 2.0 ** -20, 2.0 ** 20, 57344.0 / 7.0, 1.0 / 3.0, 1e-30, 3e30]:
        mine = quantize_values(x, scale, fmt)
        prod = xf * torch.tensor(scale, dtype=torch.float32)          # float32 multiply
        ref = torch.clamp(prod, -FMAX[fmt], FMAX[fmt]).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        assert np.array_equal(mine[finite], ref[finite]), scale
    # infinities saturate, NaN keeps its sign with mantissa all ones
    nan_pos = (x & 0x7F80 == 0x7F80) & (x & 0x7F != 0)
    got = quantize_values(x, 1.0, fmt)
    assert np.all(got[nan_pos] & 0x7F == 0x7F)
    assert np.array_equal(got[nan_pos] >> 7, (x[nan_pos] >> 15).astype(np.uint8))
    top = 0x7E if fmt == E4M3 else 0x7B
    assert got[0x7F80] == top and got[0xFF80] == top | 0x80


def test_tiny_doubling_closed_form():
    """Tiny workload: X_t = 2^t X_0 with a length-4 history over 3 steps.

    Step 0 uses the initial scale 1 and publishes s1 = fl32(448 / a0).  The
    window maximum doubles each step, so s_{t+1} = s1 * 2^-t exactly, and the
    products X_2 * s_2 equal X_1 * s_1 bit for bit, so the codes repeat."""
    x0 = bf16_normal((64, 64), 0)
    a0 = amax(x0)
    r = ring_init(4, E4M3, 1.0)
    codes = []
    xs = []
    for t in range(3):
        xt = (bf16_to_f32(x0) * np.float32(2.0 ** t)).astype(np.float32)
        xt_bits = (xt.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(bf16_to_f32(xt_bits), xt)     # doubling is exact in bf16
        xs.append(xt_bits)
        c, r = quantize_step(r, xt_bits)
        codes.append(c)
        s1 = np.float32(448.0) / a0
        assert r.scale == np.float32(s1 * np.float32(2.0 ** -t)), t
        assert r.idx == t + 1
        assert r.hist[t] == np.float32(a0 * 2 ** t)
        assert r.amax_last == np.float32(a0 * 2 ** t)
    assert np.array_equal(codes[1], codes[2])
    # step 0 used scale 1: codes are the plain casts of x0, reciprocal 1
    # step 1 used s1: the saturated codes are exactly the |x * s1| >= 432 elements
    v1 = np.abs(bf16_to_f32(xs[1]) * (np.float32(448.0) / a0))
    top = (codes[1] & 0x7F) == 0x7E
    assert np.array_equal(top, v1 >= 432.0)
    assert top.sum() >= 1


def test_window_wraps_and_keeps_last_hist_len_values():
    """Length-4 history, 10 steps with amax_t = 2^(t mod 5): the published
    scale is 448 / max(amax over the last min(t+1, 4) steps)."""
    r = ring_init(4, E4M3, 1.0)
    amaxes = []
    for t in range(10):
        a_t = 2.0 ** (t % 5)
        x = bf16_from_float([0.5, -a_t, 0.25, 0.0])
        _, r = quantize_step(r, x)
        amaxes.append(a_t)
        window = amaxes[max(0, t - 3):]
        assert r.scale == np.float32(448.0 / max(window)), t
        assert r.hist[t % 4] == np.float32(a_t)
        assert r.idx == (t + 1) % 4


def test_scale_snapshot_does_not_leak_ratio():
    """Two steps of the delayed recipe whose amax differs: the reciprocal recorded by a
    step is that of the scale the step applied, so dequantizing with it gives
    back the inputs to within the format's half-ulp, while the published
    (next) scale differs by the amax ratio."""
    x = bf16_normal((4096,), 7, 1.0)
    y = (bf16_to_f32(x) * np.float32(3.0)).astype(np.float32)
    y_bits = (y.view(np.uint32) >> 16).astype(np.uint16)
    y = bf16_to_f32(y_bits)
    r = ring_init(16, E4M3, 1.0)
    _, r = quantize_step(r, x)
    s_after_x = r.scale
    q, r = quantize_step(r, y_bits)
    assert r.scale_inv_used == np.float32(1.0) / s_after_x
    assert r.scale != s_after_x
    deq = decode_fp8(q, E4M3) * np.float64(r.scale_inv_used)
    big = np.abs(y) * np.float64(s_after_x) >= 2.0 ** -6          # normal range of E4M3
    sat = np.abs(y) * np.float64(s_after_x) > 448.0
    ok = big & ~sat
    rel = np.abs(deq[ok] - y[ok]) / np.abs(y[ok])
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_all_zero_tensor_keeps_scale():
    r = ring_init(4, E5M2, 2.0)
    _, r2 = quantize_step(r, np.zeros(100, np.uint16))
    assert r2.scale == np.float32(2.0)
    assert r2.scale_inv_used == np.float32(0.5)
    assert r2.hist[0] == 0 and r2.idx == 1


def test_nonfinite_window_keeps_scale():
    r = ring_init(2, E4M3, 1.0)
    _, r = quantize_step(r, bf16_from_float([1.0, 2.0]))
    s = r.scale
    _, r = quantize_step(r, bf16_from_float([np.inf, 1.0]))
    assert r.scale == s and np.isinf(r.hist[1])
    _, r = quantize_step(r, np.array([0x7FC0, 0x3F80], np.uint16))
    assert r.scale == s and np.isnan(r.hist[0])


def test_scale_overflow_keeps_scale():
    # window max = smallest bf16 subnormal: 448 / 2^-133 overflows binary32
    r = ring_init(1, E4M3, 1.0)
    _, r = quantize_step(r, np.array([0x0001, 0x0000], np.uint16))
    assert r.scale == np.float32(1.0)
    assert r.hist[0] == np.float32(2.0 ** -133)


def test_empty_tensor_leaves_ring_unchanged():
    r = ring_init(4, E4M3, 3.0)
    q, r2 = quantize_step(r, np.zeros(0, np.uint16))
    assert q.size == 0
    assert r2.scale == r.scale and r2.idx == r.idx and r2.scale_inv_used == r.scale_inv_used


def test_amax_is_taken_before_the_cast():
    """Regression named by the pages: with the amax of the quantized values the
    scale collapses towards 1.  Taking it on the inputs, N(0,1) data publish a
    scale near 448 / 4.5 instead."""
    x = bf16_normal((8192,), 9)
    r = ring_init(16, E4M3, 1.0)
    _, r = quantize_step(r, x)
    _, r = quantize_step(r, x)
    assert 60.0 < r.scale < 200.0
    assert r.scale == np.float32(448.0) / amax(x)
