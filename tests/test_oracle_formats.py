"""Pins of oracle/formats.py against the format definitions, torch's own
float8/bf16 casts (a library, not the oracle), hand-derived cases and brute
force.  CPU only."""
import numpy as np
import pytest
import torch

from conftest import read_golden
from oracle import E4M3, E5M2, FMAX, bf16_to_f32, bf16_ulp, decode_fp8, encode_fp8, f64_to_bf16

TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
FMT = {"e4m3": E4M3, "e5m2": E5M2}


def torch_decode(fmt):
    return torch.arange(256, dtype=torch.uint8).view(TORCH_DT[fmt]).double().numpy()


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_decode_all_256_codes_match_torch(fmt):
    mine = decode_fp8(np.arange(256, dtype=np.uint8), fmt)
    ref = torch_decode(fmt)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_format_maxima():
    assert FMAX[E4M3] == 448.0 == torch.finfo(torch.float8_e4m3fn).max
    assert FMAX[E5M2] == 57344.0 == torch.finfo(torch.float8_e5m2).max
    assert np.nanmax(decode_fp8(np.arange(256, dtype=np.uint8), E4M3)) == 448.0
    d5 = decode_fp8(np.arange(256, dtype=np.uint8), E5M2)
    assert np.max(d5[np.isfinite(d5)]) == 57344.0


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_inverts_decode(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = decode_fp8(codes, fmt)
    fin = np.isfinite(vals)
    back = encode_fp8(vals[fin].astype(np.float32), fmt)
    assert np.array_equal(back, codes[fin])


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_midpoints_tie_to_even_and_neighbours(fmt):
    top = 0x7E if fmt == E4M3 else 0x7B
    codes = np.arange(top + 1, dtype=np.uint8)
    vals = decode_fp8(codes, fmt)
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)   # exact in float32
    assert np.array_equal(mids.astype(np.float64), (vals[1:] + vals[:-1]) / 2)
    lo_code = codes[:-1]
    hi_code = codes[1:]
    even = np.where(lo_code % 2 == 0, lo_code, hi_code)
    for sign in (1, -1):
        sgn = np.uint8(0x80) if sign < 0 else np.uint8(0)
        assert np.array_equal(encode_fp8(sign * mids, fmt), even | sgn)
        up = np.nextafter(mids, np.float32(np.inf))
        dn = np.nextafter(mids, np.float32(0))
        assert np.array_equal(encode_fp8(sign * up, fmt), hi_code | sgn)
        assert np.array_equal(encode_fp8(sign * dn, fmt), lo_code | sgn)


def _structured_f32():
    rng = np.random.default_rng(11)
    parts = [
        (rng.standard_normal(200000) * s).astype(np.float32) for s in (1e-6, 1e-3, 1, 30, 300, 1e4, 1e5)
    ]
    parts.append(rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32).view(np.float32))
    parts.append(np.array([0.0, -0.0, 1e-45, -1e-45, 3.4e38, -3.4e38], dtype=np.float32))
    v = np.concatenate(parts)
    return v[~np.isnan(v)]


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_encode_matches_torch_clamp_then_cast(fmt):
    # torch's CPU float8 casts are nearest-even but not saturating, so clamping
    # to the format maximum first gives the saturating cast.
    v = _structured_f32()
    ref = torch.clamp(torch.from_numpy(v), -FMAX[fmt], FMAX[fmt]).to(TORCH_DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(encode_fp8(v, fmt), ref)


def test_encode_nan_and_inf():
    nan = np.float32(np.nan)
    assert encode_fp8(np.array([nan, -nan, np.inf, -np.inf], np.float32), E4M3).tolist() == [0x7F, 0xFF, 0x7E, 0xFE]
    assert encode_fp8(np.array([nan, -nan, np.inf, -np.inf], np.float32), E5M2).tolist() == [0x7F, 0xFF, 0x7B, 0xFB]


def test_golden_encode_cases():
    for fmt, val, code in read_golden("fp8_encode_cases.txt"):
        v = np.float32(float(val))
        got = int(encode_fp8(np.array([v], np.float32), FMT[fmt])[0])
        assert got == int(code, 16), (fmt, val, hex(got), code)


def test_bf16_to_f32_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(mine.view(np.uint32), ref.view(np.uint32))


def _all_finite_bf16_sorted():
    bits = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)   # +0 .. largest finite
    return bits, bf16_to_f32(bits).astype(np.float64)


def _brute_bf16(y):
    """Nearest finite bf16 by exhaustive comparison with all non-negative
    finite bf16 values; ties to the even bit pattern; beyond the largest
    finite value the overflow rule of nearest-even: at or past the midpoint
    to 2^128 gives infinity."""
    bits, vals = _all_finite_bf16_sorted()
    out = []
    for x in y:
        a = abs(x)
        if a >= (2.0 - 2.0 ** -8) * 2.0 ** 127:
            b = 0x7F80
        else:
            d = np.abs(vals - a)
            best = np.flatnonzero(d == d.min())
            b = int(bits[best[0]]) if len(best) == 1 else int(bits[best][bits[best] % 2 == 0][0])
        if np.signbit(x):
            b |= 0x8000
        out.append(b)
    return np.array(out, dtype=np.uint16)


def test_f64_to_bf16_brute_force():
    rng = np.random.default_rng(3)
    _, vals = _all_finite_bf16_sorted()
    pick = rng.integers(1, len(vals) - 1, 400)
    mids = (vals[pick] + vals[pick + 1]) / 2
    y = np.concatenate([
        rng.standard_normal(300) * 10.0 ** rng.integers(-30, 30, 300),
        mids, -mids, np.nextafter(mids, np.inf), np.nextafter(mids, 0),
        vals[pick], [0.0, -0.0, 1e-45, 2.0 ** -134, 3.39e38, 3.3961775292304597e38],
    ])
    assert np.array_equal(f64_to_bf16(y), _brute_bf16(y))


def test_f64_to_bf16_agrees_with_torch_on_float32_inputs():
    # A float32 value rounds once either way, so torch's float32 -> bf16 cast pins it.
    rng = np.random.default_rng(4)
    v = rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16(v.astype(np.float64)), ref)


def test_f64_to_bf16_special():
    out = f64_to_bf16(np.array([np.inf, -np.inf, np.nan, 1e300, -1e300]))
    assert out.tolist() == [0x7F80, 0xFF80, 0x7FC0, 0x7F80, 0xFF80]


def test_golden_bf16_rounding():
    for val, bits in read_golden("bf16_round_cases.txt"):
        got = int(f64_to_bf16(np.array([float(val)]))[0])
        assert got == int(bits, 16), (val, hex(got), bits)


def test_bf16_ulp_is_gap_to_next_pattern():
    bits = np.arange(0x0000, 0x7F7F, 7, dtype=np.uint32).astype(np.uint16)
    nxt = bf16_to_f32((bits + 1).astype(np.uint16)).astype(np.float64)
    cur = bf16_to_f32(bits).astype(np.float64)
    ulp = bf16_ulp(bits)
    # the next bf16 above a non-negative value lies one ulp of that value away,
    # also at the top of a binade
    assert np.array_equal(nxt - cur, ulp)
    assert bf16_ulp(np.array([0x3F80], np.uint16))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([0x0000], np.uint16))[0] == 2.0 ** -133
