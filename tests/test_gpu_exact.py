"""GEMM cases whose every output is one product, so the HIP kernel must match
the oracle bit for bit, not just within the tolerance:

* identity GEMMs that send every finite code of both formats through each
  operand position, in each layout, with unit scales and with scales whose
  product is a short binary fraction (every dequantized product then has at
  most 6 significant bits and is exact in fp32 and in bf16);
* one-hot GEMMs that pin where each (m, k) and (k, n) element lands in the
  matrix-core fragments: A[m, k] = 1 only at k = p(m), so C[m, n] = B[p(m), n]
  picks one element of B by position, for one 32 x 32 x 64 tile (a single
  matrix instruction) and for several K stages and tiles.

A flushed subnormal, a misdecoded exponent or a permuted lane shows up as a
wrong bit pattern here, where the tolerance of a long dot product could hide
it.  (Page: AstrAI history of csrc/kernels/fp8/gemm.cuh @5e76fbd1, test entry
running one matrix instruction and the GEMM layouts over several K tiles
against a CPU reference.)"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, require_gpu, say, to_dev_u8
from test_gpu_gemm import FINITE, scale_tensor

pytestmark = pytest.mark.gpu

ONE = {oracle.E4M3: 0x38, oracle.E5M2: 0x3C}      # the code of 1.0 in each format
TILES = ["auto", "256x256", "128x128", "64x64", "256x256w8", "128x128u", "64x64u"]
SCALES = [(1.0, 1.0), (0.75, 0.125)]               # alpha 1 and 0.09375 = 3 * 2^-5


def stored(logical, layout, which):
    """Stored array of a logical operand: A [M, K] is stored as A^T for TN;
    B [K, N] is stored as B^T for NT."""
    if which == "a":
        return np.ascontiguousarray(logical.T if layout == oracle.TN else logical)
    return np.ascontiguousarray(logical.T if layout == oracle.NT else logical)


def run(ds, a_log, b_log, fa, fb, layout, sa, sb, tile):
    m, k = a_log.shape
    n = b_log.shape[1]
    a, b = stored(a_log, layout, "a"), stored(b_log, layout, "b")
    lda = m if layout == oracle.TN else k
    ldb = k if layout == oracle.NT else n
    y = ds.fp8_mm(to_dev_u8(a), to_dev_u8(b), fa, fb, layout, m, n, k, scale_tensor(sa), scale_tensor(sb),
                  tile=None if tile == "auto" else tile)
    torch.cuda.synchronize()
    _, ref = oracle.mm(a, b, fa, fb, layout, m, n, k, lda, ldb, sa, sb)
    return bf16_bits(y).reshape(m, n), ref[0]


def all_codes_matrix(fmt, rows, cols):
    """rows x cols codes, each row a cyclic shift of the format's finite codes
    (every code appears in every row and, for rows >= their count, in every
    column)."""
    codes = FINITE[fmt]
    i = np.arange(rows)[:, None] + np.arange(cols)[None, :]
    return codes[i % len(codes)].astype(np.uint8)


def identity(fmt, size):
    eye = np.zeros((size, size), np.uint8)
    eye[np.arange(size), np.arange(size)] = ONE[fmt]
    return eye


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_every_code_through_each_operand(layout, tile):
    ds = require_gpu()
    lay = {"NT": oracle.NT, "NN": oracle.NN, "TN": oracle.TN}[layout]
    size = 256
    for fa, fb in [(0, 0), (1, 0), (0, 1), (1, 1)]:
        for sa, sb in SCALES:
            say(f"every code {layout} tile={tile} fa={fa} fb={fb} scales={sa},{sb}")
            # codes in A, identity B: C = dec(A) * alpha
            codes_a = all_codes_matrix(fa, size, size)
            got, ref = run(ds, codes_a, identity(fb, size), fa, fb, lay, sa, sb, tile)
            assert np.array_equal(got, ref), ("codes in A", layout, tile, fa, fb, sa,
                                              np.argwhere(got != ref)[:4].tolist())
            # identity A, codes in B: C = dec(B) * alpha
            codes_b = all_codes_matrix(fb, size, size)
            got, ref = run(ds, identity(fa, size), codes_b, fa, fb, lay, sa, sb, tile)
            assert np.array_equal(got, ref), ("codes in B", layout, tile, fa, fb, sa,
                                              np.argwhere(got != ref)[:4].tolist())


def one_hot_case(fa, fb, m, n, k, shift, stride, seed):
    """A[m, p(m)] = 1.0 with p(m) = (stride * m + shift) mod k; B holds finite
    codes drawn per position, so C[m, n] = B[p(m), n] names the element."""
    rng = np.random.default_rng(seed)
    a = np.zeros((m, k), np.uint8)
    p = (stride * np.arange(m) + shift) % k
    a[np.arange(m), p] = ONE[fa]
    b = FINITE[fb][rng.integers(0, len(FINITE[fb]), (k, n))].astype(np.uint8)
    return a, b


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_single_matrix_instruction_fragment_layout(layout):
    """32 x 32 x 64: one matrix instruction per output tile (the 64x64 tile's
    waves each run one).  Every output selects one B element by position, so
    a wrong lane or K mapping of either fragment, or a wrong accumulator lane,
    gives a wrong value."""
    ds = require_gpu()
    lay = {"NT": oracle.NT, "NN": oracle.NN, "TN": oracle.TN}[layout]
    for fa, fb in [(0, 0), (1, 0)]:
        for shift, stride in [(0, 1), (5, 1), (0, 3), (17, 7), (63, 5)]:
            say(f"single MFMA {layout} fa={fa} fb={fb} shift={shift} stride={stride}")
            a, b = one_hot_case(fa, fb, 32, 32, 64, shift, stride, 100 + shift)
            for tile in ("64x64", "auto"):
                got, ref = run(ds, a, b, fa, fb, lay, 1.0, 1.0, tile)
                assert np.array_equal(got, ref), (layout, fa, shift, stride, tile,
                                                  np.argwhere(got != ref)[:4].tolist())
            # the transposed selection: B one-hot, A drawn per position
            bt, at = one_hot_case(fb, fa, 32, 32, 64, shift, stride, 200 + shift)
            got, ref = run(ds, np.ascontiguousarray(at.T), np.ascontiguousarray(bt.T), fa, fb, lay, 1.0, 1.0,
                           "64x64")
            assert np.array_equal(got, ref), (layout, "B one-hot", shift, stride)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("tile", TILES)
def test_one_hot_over_k_stages_and_tiles(layout, tile):
    """The same selection over several K stages (K = 64 .. 448, and a K tail
    of 16 past the last whole stage) and output tiles (304 x 208, ragged against
    every tile of the family), so every stage's staging buffer and every tile's place in C is
    pinned by position."""
    ds = require_gpu()
    lay = {"NT": oracle.NT, "NN": oracle.NN, "TN": oracle.TN}[layout]
    for k in (64, 192, 448, 464):
        say(f"one-hot {layout} tile={tile} k={k}")
        a, b = one_hot_case(0, 1, 304, 208, k, 11, 37, k)
        got, ref = run(ds, a, b, 0, 1, lay, 0.75, 0.125, tile)
        assert np.array_equal(got, ref), (layout, tile, k, np.argwhere(got != ref)[:4].tolist())
