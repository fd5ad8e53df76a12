"""Pins of oracle/gemm.py: exact rational brute force on tiny problems (its
own index arithmetic per layout), integer-exact special cases, identity and
zero operands, K = 1, batch broadcast and layout equivalence.  CPU only."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import E4M3, E5M2, NN, NT, TN, bf16_to_f32, decode_fp8, mm, mm_entries
from synth import bf16_normal, random_codes

FINITE = {
    E4M3: [c for c in range(256) if (c & 0x7F) != 0x7F],
    E5M2: [c for c in range(256) if (c & 0x7C) != 0x7C],
}
E4M3_SMALL_INT = [0x00, 0x38, 0x40, 0xB8, 0xC0]       # 0, 1, 2, -1, -2


def exact_value(code, fmt):
    """Exact rational value of a finite code, from the bit fields."""
    if fmt == E4M3:
        s, e, m = code >> 7, (code >> 3) & 15, code & 7
        mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    else:
        s, e, m = code >> 7, (code >> 2) & 31, code & 3
        mag = Fraction(m, 4) * Fraction(2) ** -14 if e == 0 else (1 + Fraction(m, 4)) * Fraction(2) ** (e - 15)
    return -mag if s else mag


def nearest_bf16_exact(q):
    """Nearest bf16 to an exact rational, ties to even, by scanning the
    representable values of q's binade (bf16 has 8 significant bits)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    step = Fraction(2) ** (e - 7)
    n = a / step
    lo = n.numerator // n.denominator
    rem = n - lo
    r = lo + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1) else lo
    val = r * step
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(val))
    assert Fraction(float(f)) == val
    return sign | int(f.view(np.uint32) >> 16)


def brute_mm(a, b, fa, fb, layout, m, n, k, lda, ldb, sa, sb, bias, batch, stra, strb):
    out = np.zeros((batch, m, n), dtype=np.uint16)
    sa_q, sb_q = Fraction(float(np.float32(sa))), Fraction(float(np.float32(sb)))
    for bi in range(batch):
        for i in range(m):
            for j in range(n):
                acc = Fraction(0)
                for kk in range(k):
                    ia = bi * stra + (kk * lda + i if layout == TN else i * lda + kk)
                    ib = bi * strb + (j * ldb + kk if layout == NT else kk * ldb + j)
                    acc += exact_value(int(a[ia]), fa) * exact_value(int(b[ib]), fb)
                y = acc * sa_q * sb_q
                if bias is not None:
                    y += Fraction(float(bf16_to_f32(bias[j:j + 1])[0]))
                out[bi, i, j] = nearest_bf16_exact(y)
    return out


def operand_size(layout, which, m, n, k, ld, batch, stride):
    rows = {(NT, "a"): m, (NN, "a"): m, (TN, "a"): k, (NT, "b"): n, (NN, "b"): k, (TN, "b"): k}[(layout, which)]
    return stride * (batch - 1) + rows * ld


@pytest.mark.parametrize("layout", [NT, NN, TN])
@pytest.mark.parametrize("fa,fb", [(E4M3, E4M3), (E5M2, E4M3)])
def test_exact_rational_brute_force(layout, fa, fb):
    rng = np.random.default_rng(100 + layout + 10 * fa)
    m, n, k, batch = 5, 7, 13, 2
    lda = (k if layout != TN else m) + 3
    ldb = (k if layout == NT else n) + 2
    stra = lda * (m if layout != TN else k) + 5
    strb = 0 if layout == NN else ldb * (n if layout == NT else k) + 1
    a = random_codes(operand_size(layout, "a", m, n, k, lda, batch, stra), 1, FINITE[fa])
    b = random_codes(operand_size(layout, "b", m, n, k, ldb, batch, strb), 2, FINITE[fb])
    # keep products in a modest range so the result stays finite in bf16
    sa, sb = np.float32(rng.uniform(0.001, 0.01)), np.float32(rng.uniform(0.5, 2))
    bias = bf16_normal((n,), 3)
    y, out = mm(a, b, fa, fb, layout, m, n, k, lda, ldb, sa, sb, bias, batch, stra, strb)
    ref = brute_mm(a, b, fa, fb, layout, m, n, k, lda, ldb, sa, sb, bias, batch, stra, strb)
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("layout", [NT, NN, TN])
def test_small_integer_products_are_exact(layout):
    # entries in {-2,-1,0,1,2}, K <= 64: every sum is an integer of magnitude
    # <= 256, exactly representable in bf16
    m, n, k = 33, 17, 64
    a = random_codes((m * k,), 5, E4M3_SMALL_INT)
    b = random_codes((n * k,), 6, E4M3_SMALL_INT)
    lda = k if layout != TN else m
    ldb = k if layout == NT else n
    _, out = mm(a, b, E4M3, E4M3, layout, m, n, k, lda, ldb, 1.0, 1.0)
    ia = {NT: lambda i, kk: i * lda + kk, NN: lambda i, kk: i * lda + kk, TN: lambda i, kk: kk * lda + i}[layout]
    ib = {NT: lambda j, kk: j * ldb + kk, NN: lambda j, kk: kk * ldb + j, TN: lambda j, kk: kk * ldb + j}[layout]
    val = {0x00: 0, 0x38: 1, 0x40: 2, 0xB8: -1, 0xC0: -2}
    for i in range(m):
        for j in range(n):
            s = sum(val[int(a[ia(i, kk)])] * val[int(b[ib(j, kk)])] for kk in range(k))
            assert bf16_to_f32(out[0, i, j:j + 1])[0] == s


def test_identity_zero_and_k1():
    n, k = 24, 16
    b = random_codes((n * k,), 8, FINITE[E4M3])
    eye = np.zeros((k, k), np.uint8)
    np.fill_diagonal(eye, 0x38)                     # 1.0
    sb = np.float32(0.37)
    _, out = mm(eye.reshape(-1), b, E4M3, E4M3, NT, k, n, k, k, k, 1.0, sb)
    bm = decode_fp8(b.reshape(n, k), E4M3).T        # B[k, n]
    expect = bm * np.float64(sb)
    assert np.array_equal(bf16_to_f32(out[0]), np.array([[np.float32(0)]]) + _round(expect))
    bias = bf16_normal((n,), 9)
    _, out0 = mm(np.zeros(k * k, np.uint8), b, E4M3, E4M3, NT, k, n, k, k, k, 3.0, sb, bias)
    assert np.array_equal(out0[0], np.broadcast_to(bias, (k, n)))
    _, outk0 = mm(np.zeros(0, np.uint8), np.zeros(0, np.uint8), E4M3, E4M3, NT, 3, n, 0, 1, 1, 1.0, 1.0, bias)
    assert np.array_equal(outk0[0], np.broadcast_to(bias, (3, n)))
    a1 = random_codes((5,), 10, FINITE[E5M2])
    b1 = random_codes((n,), 11, FINITE[E4M3])
    y, _ = mm(a1, b1, E5M2, E4M3, NN, 5, n, 1, 1, n, 2.0, 0.5, bias)
    exp1 = decode_fp8(a1, E5M2)[:, None] * decode_fp8(b1, E4M3)[None, :] * 1.0 + bf16_to_f32(bias)[None, :]
    assert np.array_equal(y[0], exp1)


def _round(x):
    from oracle import f64_to_bf16
    return bf16_to_f32(f64_to_bf16(x)).astype(np.float64)


def test_batch_broadcast_matches_per_batch_calls():
    m, n, k, batch = 9, 11, 20, 4
    a = random_codes((batch * m * k,), 12, FINITE[E4M3])
    b = random_codes((n * k,), 13, FINITE[E4M3])
    y, out = mm(a, b, E4M3, E4M3, NT, m, n, k, k, k, 0.01, 0.02, None, batch, m * k, 0)
    for bi in range(batch):
        y1, out1 = mm(a[bi * m * k:(bi + 1) * m * k], b, E4M3, E4M3, NT, m, n, k, k, k, 0.01, 0.02)
        assert np.array_equal(out[bi], out1[0]) and np.array_equal(y[bi], y1[0])


def test_layouts_agree_on_the_same_logical_product():
    m, n, k = 19, 23, 40
    am = random_codes((m, k), 14, FINITE[E4M3])      # logical A [M, K]
    bm = random_codes((k, n), 15, FINITE[E4M3])      # logical B [K, N]
    _, nt = mm(am.reshape(-1), np.ascontiguousarray(bm.T).reshape(-1), E4M3, E4M3, NT, m, n, k, k, k, 0.1, 0.1)
    _, nn = mm(am.reshape(-1), bm.reshape(-1), E4M3, E4M3, NN, m, n, k, k, n, 0.1, 0.1)
    _, tn = mm(np.ascontiguousarray(am.T).reshape(-1), bm.reshape(-1), E4M3, E4M3, TN, m, n, k, m, n, 0.1, 0.1)
    assert np.array_equal(nt, nn) and np.array_equal(nn, tn)


@pytest.mark.parametrize("layout", [NT, NN, TN])
def test_entries_match_full(layout):
    m, n, k, batch = 21, 18, 50, 3
    lda = k if layout != TN else m
    ldb = k if layout == NT else n
    sa_rows = m if layout != TN else k
    sb_rows = n if layout == NT else k
    a = random_codes((batch * sa_rows * lda,), 16, FINITE[E5M2])
    b = random_codes((batch * sb_rows * ldb,), 17, FINITE[E4M3])
    bias = bf16_normal((n,), 18)
    y, out = mm(a, b, E5M2, E4M3, layout, m, n, k, lda, ldb, 0.003, 0.2, bias, batch,
                sa_rows * lda, sb_rows * ldb)
    rng = np.random.default_rng(0)
    bi, mi, ni = rng.integers(0, batch, 60), rng.integers(0, m, 60), rng.integers(0, n, 60)
    ye, oute = mm_entries(a, b, E5M2, E4M3, layout, m, n, k, lda, ldb, 0.003, 0.2, bi, mi, ni, bias,
                          sa_rows * lda, sb_rows * ldb)
    assert np.allclose(ye, y[bi, mi, ni], rtol=1e-14, atol=0)
    assert np.array_equal(oute, out[bi, mi, ni])


# ---------------------------------------------------------------------------
# The acceptance helpers every GEMM verdict goes through: oracle.tolerance and
# oracle.max_abs_dequant, against hand-derived rows (tests/golden/
# gemm_acceptance_cases.txt).  Each mutant below is a plausible slip in one of
# them; the rows must catch every one.

import math

import oracle as _oracle
from conftest import read_golden

_FMT = {"e4m3": E4M3, "e5m2": E5M2}


def _tol_rows():
    return [(int(r[1], 16), int(r[2]), float(r[3]), float(r[4]), float(r[5]))
            for r in read_golden("gemm_acceptance_cases.txt") if r[0] == "tol"]


def _mad_rows():
    out = []
    for r in read_golden("gemm_acceptance_cases.txt"):
        if r[0] != "mad":
            continue
        codes = [] if r[3] == "-" else [int(c, 16) for c in r[3].split(",")]
        out.append((_FMT[r[1]], float(r[2]), np.array(codes, dtype=np.uint8), float(r[4])))
    return out


def _tol_ok(fn):
    return all(math.isclose(float(fn(np.array([b], dtype=np.uint16), k, ma, mb)[0]), want, rel_tol=1e-12, abs_tol=0.0)
               for b, k, ma, mb, want in _tol_rows())


def _mad_ok(fn):
    return all(math.isclose(float(fn(codes, fmt, s)), want, rel_tol=1e-15, abs_tol=0.0)
               for fmt, s, codes, want in _mad_rows())


def test_tolerance_golden_rows():
    rows = _tol_rows()
    assert len(rows) >= 10
    for b, k, ma, mb, want in rows:
        got = float(_oracle.tolerance(np.array([b], dtype=np.uint16), k, ma, mb)[0])
        assert math.isclose(got, want, rel_tol=1e-12, abs_tol=0.0), (hex(b), k, ma, mb, got, want)


def test_max_abs_dequant_golden_rows():
    rows = _mad_rows()
    assert len(rows) >= 8
    for fmt, s, codes, want in rows:
        got = _oracle.max_abs_dequant(codes, fmt, s)
        assert math.isclose(got, want, rel_tol=1e-15, abs_tol=0.0), (fmt, s, codes, got, want)


def test_golden_rows_catch_tolerance_mutants():
    ulp = _oracle.bf16_ulp
    mutants = {
        "one ulp": lambda r, k, a, b: 1.0 * ulp(r) + 1e-3 * np.sqrt(k) * a * b,
        "K not rooted": lambda r, k, a, b: 2.0 * ulp(r) + 1e-3 * k * a * b,
        "one maximum dropped": lambda r, k, a, b: 2.0 * ulp(r) + 1e-3 * np.sqrt(k) * a,
        "1e-2 factor": lambda r, k, a, b: 2.0 * ulp(r) + 1e-2 * np.sqrt(k) * a * b,
        "ulp one exponent off": lambda r, k, a, b: 4.0 * ulp(r) + 1e-3 * np.sqrt(k) * a * b,
        "no subnormal floor": lambda r, k, a, b: 2.0 * np.where(
            np.abs(bf16_to_f32(r)) > 0,
            np.ldexp(1.0, np.frexp(np.where(np.abs(bf16_to_f32(r)) > 0, np.abs(bf16_to_f32(r)), 1.0))[1] - 8),
            2.0 ** -133) + 1e-3 * np.sqrt(k) * a * b,
        "ulp taken of the signed value": lambda r, k, a, b: 2.0 * np.where(bf16_to_f32(r) < 0, 0.0, ulp(r))
        + 1e-3 * np.sqrt(k) * a * b,
    }
    assert _tol_ok(lambda r, k, a, b: _oracle.tolerance(r, k, a, b))
    for name, fn in mutants.items():
        assert not _tol_ok(fn), f"the golden rows do not catch the tolerance mutant '{name}'"


def test_golden_rows_catch_max_abs_dequant_mutants():
    def present(codes):
        c = np.asarray(codes, dtype=np.uint8).reshape(-1)
        return np.unique(c)

    def signed_max(codes, fmt, s):
        v = decode_fp8(present(codes), fmt)
        return float(np.nanmax(v)) * float(np.float32(s)) if v.size else 0.0

    def no_scale(codes, fmt, s):
        v = np.abs(decode_fp8(present(codes), fmt))
        return float(np.nanmax(v)) if v.size else 0.0

    def nan_not_skipped(codes, fmt, s):
        v = np.abs(decode_fp8(present(codes), fmt))
        return float(np.max(v)) * float(np.float32(s)) if v.size else 0.0

    def scale_not_rounded(codes, fmt, s):
        v = np.abs(decode_fp8(present(codes), fmt))
        return float(np.nanmax(v)) * float(s) if v.size else 0.0

    def wrong_format(codes, fmt, s):
        v = np.abs(decode_fp8(present(codes), 1 - fmt))
        return float(np.nanmax(v)) * float(np.float32(s)) if v.size else 0.0

    def divides(codes, fmt, s):
        v = np.abs(decode_fp8(present(codes), fmt))
        return float(np.nanmax(v)) / float(np.float32(s)) if v.size else 0.0

    assert _mad_ok(_oracle.max_abs_dequant)
    with np.errstate(invalid="ignore"):
        for fn in (signed_max, no_scale, nan_not_skipped, scale_not_rounded, wrong_format, divides):
            assert not _mad_ok(fn), f"the golden rows do not catch the max_abs_dequant mutant {fn.__name__}"


def test_identity_products_are_exact_decoded_codes():
    """The premise of the GPU's bit-exact identity GEMMs: with one operand the
    identity (code of 1.0 on the diagonal) every output is one product, and
    with scales 1 or 0.75 * 0.125 each is the decoded code times the scales,
    exactly (at most 6 significant bits, so the one bf16 rounding is exact)."""
    one = {E4M3: 0x38, E5M2: 0x3C}
    for fmt in (E4M3, E5M2):
        codes = np.array(FINITE[fmt], np.uint8)
        a = codes[(np.arange(256)[:, None] + np.arange(256)[None, :]) % len(codes)]
        eye = np.zeros((256, 256), np.uint8)
        eye[np.arange(256), np.arange(256)] = one[fmt]
        for sa, sb in [(1.0, 1.0), (0.75, 0.125)]:
            want = decode_fp8(a, fmt) * sa * sb
            _, ref = mm(a, eye, fmt, fmt, NN, 256, 256, 256, 256, 256, sa, sb)
            assert np.array_equal(bf16_to_f32(ref[0]).astype(np.float64), want)
            _, ref = mm(eye, a, fmt, fmt, NN, 256, 256, 256, 256, 256, sa, sb)
            assert np.array_equal(bf16_to_f32(ref[0]).astype(np.float64), want)
