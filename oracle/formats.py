"""Number formats of the path: bf16 inputs/outputs and the two OCP 8-bit floats.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU
baseline leg of the benchmark may import this package.

Sources.  The pages (AstrAI commit history of astrai/extension/fp8.py and of
csrc/kernels/fp8/gemm.cuh) name the two formats by their roles: E4M3 for
forward operands, E5M2 for gradients, with E4M3's largest finite value 448
mentioned where the collapsed-scale bug is described (fp8.py history
@4dc5e923, amax fix entry).  They print no encoding tables.  The bit layouts
below are the OCP 8-bit floating point definitions ("e4m3fn": no infinities,
one NaN mantissa pattern; "e5m2": IEEE-like with infinities).

Readings taken where the pages are silent:
  * encoding is round-to-nearest, ties to the code with even mantissa, and
    saturating: any magnitude at or above the format maximum, infinity
    included, becomes the largest finite code of that sign;
  * a NaN encodes as 0x7F with the sign bit of the NaN (mantissa all ones);
  * the sign of zero and of values that round to zero is kept.
"""
import numpy as np

E4M3 = 0
E5M2 = 1

# Element types a quantize may read (fp8.py history @f4c44ebf, entry that
# templates the quantize on its input type: bf16, fp16 or fp32).
IN_BF16 = 0
IN_F16 = 1
IN_F32 = 2

# Largest finite magnitude: E4M3 (1 + 6/8) * 2^8 = 448, E5M2 (1 + 3/4) * 2^15.
FMAX = {E4M3: 448.0, E5M2: 57344.0}


def _check_fmt(fmt):
    if fmt not in (E4M3, E5M2):
        raise ValueError("fmt must be E4M3 (0) or E5M2 (1)")


def decode_fp8(codes, fmt):
    """Value of each 8-bit code, as float64 (exact), NaN/inf where defined.

    E4M3 (bias 7): exponent field 0 is subnormal m * 2^-9; all-ones exponent
    with all-ones mantissa is NaN; otherwise (1 + m/8) * 2^(e-7).
    E5M2 (bias 15): exponent 0 is m * 2^-16; exponent 31 is inf (m = 0) or
    NaN; otherwise (1 + m/4) * 2^(e-15).
    """
    _check_fmt(fmt)
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    if fmt == E4M3:
        e = (c >> 3) & 15
        m = c & 7
        mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
    else:
        e = (c >> 2) & 31
        m = c & 3
        mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(e - 15.0))
        mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return s * mag


def _positive_table(fmt):
    """Finite non-negative codes of the format, in increasing value order.

    For both formats the value of a non-negative code grows with the code, so
    the table is codes 0 .. largest finite code (0x7E for E4M3, 0x7B for E5M2).
    """
    top = 0x7E if fmt == E4M3 else 0x7B
    codes = np.arange(top + 1, dtype=np.uint8)
    return codes, decode_fp8(codes, fmt)


def encode_fp8(v, fmt):
    """Saturating round-to-nearest-even encoding of float32 values.

    For each finite |v| below the maximum, take the two table neighbours
    lo <= |v| < hi and keep the nearer one; on an exact tie keep the one whose
    code is even (adjacent codes alternate mantissa parity, so the even code is
    the even mantissa).  All arithmetic is on float64, where the differences
    of a float32 and an 8-bit-float value are exact.
    """
    _check_fmt(fmt)
    v = np.asarray(v, dtype=np.float32)
    flat = v.reshape(-1).astype(np.float64)
    codes, table = _positive_table(fmt)
    fmax = FMAX[fmt]
    a = np.abs(flat)
    nan = np.isnan(flat)
    a_safe = np.where(nan, 0.0, a)
    sat = a_safe >= fmax
    a_in = np.where(sat, 0.0, a_safe)
    i = np.searchsorted(table, a_in, side="right") - 1      # table[i] <= a < table[i+1]
    i = np.clip(i, 0, len(table) - 2)
    lo = table[i]
    hi = table[i + 1]
    d_lo = a_in - lo
    d_hi = hi - a_in
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (i % 2 == 1))
    mag_code = np.where(pick_hi, codes[i + 1], codes[i]).astype(np.uint8)
    mag_code = np.where(sat, codes[-1], mag_code)
    mag_code = np.where(nan, np.uint8(0x7F), mag_code)
    sign = np.signbit(flat).astype(np.uint8) << 7
    return (mag_code | sign).astype(np.uint8).reshape(v.shape)


# ---------------------------------------------------------------------------
# bf16

def bf16_to_f32(bits):
    """bf16 bit patterns (uint16) to float32: the upper half of the binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f64_to_bf16(y):
    """Round float64 values straight to bf16 (uint16 bits), nearest-even.

    bf16 keeps 8 significant bits; a finite value in [2^E, 2^(E+1)) is rounded
    to a multiple of 2^(E-7), with E floored at -126 so that the subnormal
    range keeps the fixed spacing 2^-133.  A result of 2^128 or more is
    infinity (ties at the top go to the even, overflowing neighbour).  NaN
    becomes the quiet NaN 0x7FC0 with its sign.
    """
    y = np.asarray(y, dtype=np.float64)
    flat = y.reshape(-1)
    a = np.abs(flat)
    sign = np.signbit(flat)
    nan = np.isnan(flat)
    inf = np.isinf(flat)
    fin = ~(nan | inf) & (a > 0)
    a_f = np.where(fin, a, 1.0)
    _, ex = np.frexp(a_f)                       # a = f * 2^ex, f in [0.5, 1)
    big_e = np.maximum(ex - 1, -126)
    ulp = np.ldexp(1.0, big_e - 7)
    r = np.rint(a_f / ulp) * ulp                # exact scaling, ties to even
    r = np.where(fin, r, 0.0)
    over = r >= 2.0 ** 128
    r32 = np.where(over, 0.0, r).astype(np.float32)   # exact: r has <= 8 bits
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(over | inf, np.uint16(0x7F80), bits)
    bits = np.where(nan, np.uint16(0x7FC0), bits)
    bits = bits | (sign.astype(np.uint16) << np.uint16(15))
    return bits.astype(np.uint16).reshape(y.shape)


def input_to_f32(bits, kind):
    """float32 values of input elements given as raw bits: bf16 and fp16
    (uint16 patterns) widen exactly, fp32 (uint32 patterns) is reinterpreted."""
    if kind == IN_BF16:
        return bf16_to_f32(bits)
    if kind == IN_F16:
        return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)
    if kind == IN_F32:
        return np.asarray(bits, dtype=np.uint32).view(np.float32)
    raise ValueError("kind must be IN_BF16, IN_F16 or IN_F32")


def bf16_ulp(bits):
    """Spacing of bf16 numbers at each given bf16 value (float64).

    2^(max(floor(log2|r|), -126) - 7); for r = 0 the subnormal spacing 2^-133.
    """
    r = np.abs(bf16_to_f32(bits).astype(np.float64))
    r_safe = np.where((r > 0) & np.isfinite(r), r, 1.0)
    _, ex = np.frexp(r_safe)
    e = np.where((r > 0) & np.isfinite(r), np.maximum(ex - 1, -126), -126)
    return np.ldexp(1.0, e - 7)
