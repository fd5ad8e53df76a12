"""Pins of the oracle's backward-neighbour, dynamic-recipe, input-type and
8-bit-bias functions: library casts over every fp16 pattern, brute-force
index loops for the two quantize orientations, exact integer and rational
column sums, closed forms of the dynamic scale.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import (DUAL, E4M3, E5M2, FMAX, IN_BF16, IN_F16, IN_F32, OUT_BF16, OUT_F32, ROWWISE,
                    TRANSPOSED, advance_ring, amax, bias_grad, bias_grad_tolerance, decode_fp8,
                    dynamic_ring_after, dynamic_scale, f64_to_bf16, input_to_f32, quantize_dynamic,
                    quantize_step, quantize_step_2d, quantize_values, ring_init)
from synth import bf16_from_float, bf16_normal, random_codes

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}


def f32_bits(x):
    return int(np.float32(x).view(np.uint32))


# ---------------------------------------------------------------------------
# input types

def test_fp16_widening_every_pattern_matches_torch():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = input_to_f32(h, IN_F16)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.float16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_fp16_every_pattern_against_torch(fmt):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    xf = torch.from_numpy(h.view(np.int16)).view(torch.float16).float()
    finite = torch.isfinite(xf).numpy()
    for scale in [1.0, 448.0 / 3.25, 2.0 ** -10, 2.0 ** 12, 1.0 / 3.0]:
        mine = quantize_values(h, scale, fmt, IN_F16)
        ref = torch.clamp(xf * torch.tensor(scale, dtype=torch.float32), -FMAX[fmt], FMAX[fmt])
        ref = ref.to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        assert np.array_equal(mine[finite], ref[finite]), scale
    nan = np.isnan(xf.numpy())
    got = quantize_values(h, 1.0, fmt, IN_F16)
    assert np.all(got[nan] & 0x7F == 0x7F)
    assert np.array_equal(got[nan] >> 7, (h[nan] >> 15).astype(np.uint8))


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_quantize_fp32_against_torch(fmt):
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 300,
                        np.float32(2.0) ** rng.integers(-140, 20, 50000).astype(np.float32),
                        np.array([0.0, -0.0, 448.0, 464.0, -465.0, 57344.0, 61440.0, 1e-45], np.float32)])
    bits = v.view(np.uint32)
    for scale in [1.0, 0.37, 2.0 ** 30]:
        mine = quantize_values(bits, scale, fmt, IN_F32)
        prod = torch.from_numpy(v) * torch.tensor(scale, dtype=torch.float32)
        ref = torch.clamp(prod, -FMAX[fmt], FMAX[fmt]).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
        ok = np.isfinite(prod.numpy())
        assert np.array_equal(mine[ok], ref[ok]), scale


def test_amax_input_types():
    v = np.array([1.5, -7.25, 3.0, -0.0], np.float32)
    assert amax(v.view(np.uint32), IN_F32) == np.float32(7.25)
    h = v.astype(np.float16).view(np.uint16)
    assert amax(h, IN_F16) == np.float32(7.25)
    h_nan = np.concatenate([h, np.array([0x7E01], np.uint16)])
    assert np.isnan(amax(h_nan, IN_F16))
    big = np.array([65504.0, -1.0], np.float16).view(np.uint16)
    assert f32_bits(amax(big, IN_F16)) == f32_bits(65504.0)


# ---------------------------------------------------------------------------
# quantize in two orientations

@pytest.mark.parametrize("layout", [ROWWISE, TRANSPOSED, DUAL])
def test_orientations_are_the_plain_codes_by_index(layout):
    rows, cols = 5, 7
    x = bf16_normal((rows, cols), 21, 3.0, outliers=True)
    ring = ring_init(4, E4M3, 2.5)
    y, y_t, r2 = quantize_step_2d(ring, x, rows, cols, layout)
    flat, r1 = quantize_step(ring, x.reshape(-1))
    for r in range(rows):
        for c in range(cols):
            want = flat[r * cols + c]
            if y is not None:
                assert y[r, c] == want
            if y_t is not None:
                assert y_t[c, r] == want
    assert (y is None) == (layout == TRANSPOSED) and (y_t is None) == (layout == ROWWISE)
    assert f32_bits(r1.scale) == f32_bits(r2.scale) and r1.idx == r2.idx
    assert np.array_equal(r1.hist.view(np.uint32), r2.hist.view(np.uint32))


# ---------------------------------------------------------------------------
# bias gradient

def test_bias_grad_small_integers_exact():
    rows, cols = 37, 11
    rng = np.random.default_rng(3)
    ints = rng.integers(-8, 9, size=(rows, cols))
    g = bf16_from_float(ints.astype(np.float32))
    s, bits, f = bias_grad(g, rows, cols, IN_BF16)
    for c in range(cols):
        exact = int(sum(int(ints[r, c]) for r in range(rows)))
        assert s[c] == exact and f[c] == exact
        assert oracle.bf16_to_f32(bits[c:c + 1])[0] == np.float32(exact)     # |sum| <= 296 is exact in bf16


def test_bias_grad_rational_brute_force_and_rounding():
    rows, cols = 9, 4
    g = bf16_normal((rows, cols), 8, 1e-3)
    vals = oracle.bf16_to_f32(g).astype(np.float64)
    s, bits, f = bias_grad(g, rows, cols, IN_BF16)
    for c in range(cols):
        exact = sum(Fraction(float(vals[r, c])) for r in range(rows))
        assert Fraction(float(s[c])) == exact                   # 9 bf16 values sum exactly in float64
        assert bits[c] == f64_to_bf16(np.array([float(exact)]))[0]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_bias_grad_of_codes_dequantizes_in_float32(fmt):
    rows, cols = 6, 5
    codes = random_codes((rows, cols), 4, np.array([c for c in range(256) if (c & 0x7F) < 0x70], np.uint8))
    s_inv = np.float32(0.0123)
    s, _, _ = bias_grad(codes, rows, cols, None, fmt, s_inv)
    for c in range(cols):
        want = 0.0
        for r in range(rows):
            want += float(np.float32(np.float32(decode_fp8(codes[r, c], fmt)) * s_inv))
        assert abs(s[c] - want) <= 1e-15 * max(1.0, abs(want))


def test_bias_grad_tolerance_covers_float32_summation():
    rows, cols = 4096, 64
    g = bf16_normal((rows, cols), 9, 1.0, outliers=True)
    s, bits, f = bias_grad(g, rows, cols, IN_BF16)
    seq = np.zeros(cols, np.float32)
    for r in range(rows):                                   # sequential float32 sums, then one rounding
        seq = (seq + oracle.bf16_to_f32(g[r])).astype(np.float32)
    for out_kind, ref in [(OUT_F32, f), (OUT_BF16, bits)]:
        got = seq if out_kind == OUT_F32 else oracle.f64_to_bf16(seq.astype(np.float64))
        gv = got.astype(np.float64) if out_kind == OUT_F32 else oracle.bf16_to_f32(got).astype(np.float64)
        rv = ref.astype(np.float64) if out_kind == OUT_F32 else oracle.bf16_to_f32(ref).astype(np.float64)
        tol = bias_grad_tolerance(g, rows, cols, IN_BF16, ref, out_kind)
        assert np.all(np.abs(gv - rv) <= tol)


# ---------------------------------------------------------------------------
# dynamic recipe

@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_dynamic_scale_closed_form(fmt):
    base = np.array([1.75, -0.5, 0.25, 1.0, -1.75, 0.0], np.float32)
    for k in [-20, -3, 0, 5]:
        x = bf16_from_float(base * np.float32(2.0 ** k))
        codes, s, s_inv, a = quantize_dynamic(x, fmt)
        assert a == np.float32(1.75 * 2.0 ** k)
        assert s == np.float32(FMAX[fmt] / 1.75 * 2.0 ** -k)            # a power of two times 256 or 32768
        top = 0x7E if fmt == E4M3 else 0x7B
        assert codes[0] == top and codes[4] == top | 0x80               # the amax elements map to +-FMAX
        assert s_inv == np.float32(1.0) / s


def test_dynamic_degenerate_tensors_use_scale_one():
    for vals in ([0.0, -0.0], [1.0, np.inf], [np.nan, 2.0]):
        x = bf16_from_float(np.array(vals, np.float32))
        _, s, s_inv, _ = quantize_dynamic(x, E4M3)
        assert s == np.float32(1.0) and s_inv == np.float32(1.0)
    assert dynamic_scale(np.float32(1e-44), E4M3) == np.float32(1.0)   # 448 / 1e-44 overflows float32


def test_dynamic_ring_is_a_length_one_delayed_ring():
    x = bf16_normal((300,), 12, 2.0)
    r = dynamic_ring_after(x, E4M3)
    _, s, _, a = quantize_dynamic(x, E4M3)
    pre = ring_init(1, E4M3, float(s))                  # a length-1 ring already holding the scale
    post = advance_ring(pre, a)
    assert f32_bits(post.scale) == f32_bits(r.scale) == f32_bits(s)
    assert f32_bits(post.scale_inv_used) == f32_bits(r.scale_inv_used)
    assert post.hist[0] == r.hist[0] == a


# ---------------------------------------------------------------------------
# 8-bit bias in the GEMM

@pytest.mark.parametrize("bfmt", [E4M3, E5M2])
def test_fp8_bias_exact_rational(bfmt):
    m, n, k = 3, 5, 4
    a = random_codes((m * k,), 31, np.array([0x38, 0x40, 0xB8, 0x30], np.uint8))
    b = random_codes((n * k,), 32, np.array([0x38, 0x40, 0xB8, 0x30], np.uint8))
    bias = random_codes((n,), 33, np.array([c for c in range(256) if (c & 0x7F) < 0x70], np.uint8))
    bsi = np.float32(0.0625)
    y, out = oracle.mm(a, b, E4M3, E4M3, oracle.NT, m, n, k, k, k, 1.0, 1.0, bias=bias, bias_fmt=bfmt,
                       bias_scale_inv=bsi)
    da, db, dbias = decode_fp8(a, E4M3), decode_fp8(b, E4M3), decode_fp8(bias, bfmt)
    for i in range(m):
        for j in range(n):
            acc = sum(Fraction(float(da[i * k + t])) * Fraction(float(db[j * k + t])) for t in range(k))
            bias_f32 = Fraction(float(np.float32(np.float32(dbias[j]) * bsi)))
            assert Fraction(float(y[0, i, j])) == acc + bias_f32
