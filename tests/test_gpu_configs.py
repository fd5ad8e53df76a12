"""The five workloads of the path, each run through the HIP library and the
oracle from the same seeded bf16 inputs.  Each side quantizes its own inputs
(GPU kernels vs oracle); quantized bytes and every ring field must agree bit
for bit, GEMM outputs within the tolerance of oracle.tolerance.  Full
comparisons where the float64 oracle is quick, sampled entries otherwise."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, f32_bits, require_gpu, say, to_dev_bf16
from synth import bf16_normal, bf16_normal_sequence, seed_for

pytestmark = pytest.mark.gpu
E4M3, E5M2 = oracle.E4M3, oracle.E5M2


class Side:
    """One operand's ring on both sides, stepped together."""

    def __init__(self, ds, fmt, hist_len, init_scale=1.0):
        self.ds = ds
        self.fmt = fmt
        self.ring = ds.ScaleRing(hist_len, fmt, init_scale)
        self.ref = oracle.ring_init(hist_len, fmt, init_scale)

    def quantize(self, x_bits, check_codes=True):
        """Quantize on the GPU and in the oracle; returns (device codes,
        oracle codes or None); the ring states are compared bit for bit.
        x_bits: host bf16 bit patterns, or a bf16 device tensor whose bits
        the oracle then receives copied to the host."""
        if isinstance(x_bits, torch.Tensor):
            x_dev = x_bits
            x_bits = x_dev.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            x_dev = to_dev_bf16(x_bits)
        q = self.ds.fp8_quantize(x_dev, self.fmt, self.ring)
        if check_codes:
            codes, self.ref = oracle.quantize_step(self.ref, x_bits)
        else:
            # the ring update depends on the tensor only through its amax
            codes = None
            self.ref = oracle.advance_ring(self.ref, oracle.amax(x_bits))
        torch.cuda.synchronize()
        g = self.ring.read()
        assert g["scale_bits"] == f32_bits(self.ref.scale)
        assert g["scale_inv_used_bits"] == f32_bits(self.ref.scale_inv_used)
        assert g["amax_last_bits"] == f32_bits(self.ref.amax_last)
        assert g["idx"] == self.ref.idx
        assert g["hist_bits"] == [int(v) for v in self.ref.hist.view(np.uint32)]
        assert g["amax_bits"] == 0 and g["ticket"] == 0 and g["status"] == 0 and g["group_scratch_zero"]
        if codes is not None:
            got = q.cpu().numpy()
            assert np.array_equal(got, codes), np.flatnonzero(got.reshape(-1) != codes.reshape(-1))[:8]
        return q, codes

    @property
    def s_inv(self):
        return self.ref.scale_inv_used


def check_mm(ds, out, a_codes, b_codes, fa, fb, layout, m, n, k, sa, sb, bias=None, batch=1,
             stride_a=0, stride_b=0, sample=None, what=""):
    """Compare a GPU GEMM output with the oracle, fully or on `sample`
    random entries."""
    lda = m if layout == oracle.TN else k
    ldb = k if layout == oracle.NT else n
    got = bf16_bits(out).reshape(batch, m, n)
    amax_a = oracle.max_abs_dequant(a_codes, fa, sa)
    amax_b = oracle.max_abs_dequant(b_codes, fb, sb)
    if sample is None:
        _, ref = oracle.mm(a_codes, b_codes, fa, fb, layout, m, n, k, lda, ldb, sa, sb, bias, batch,
                           stride_a, stride_b)
        g = got
    else:
        rng = np.random.default_rng(sample)
        bi, mi, ni = rng.integers(0, batch, sample), rng.integers(0, m, sample), rng.integers(0, n, sample)
        # always include the corners of the output
        bi = np.concatenate([bi, [0, batch - 1]]); mi = np.concatenate([mi, [0, m - 1]])
        ni = np.concatenate([ni, [0, n - 1]])
        _, ref = oracle.mm_entries(a_codes, b_codes, fa, fb, layout, m, n, k, lda, ldb, sa, sb, bi, mi, ni, bias,
                                   stride_a, stride_b)
        g = got[bi, mi, ni]
    err = np.abs(oracle.bf16_to_f32(g).astype(np.float64) - oracle.bf16_to_f32(ref).astype(np.float64))
    tol = oracle.tolerance(ref, k, amax_a, amax_b)
    bad = ~(err <= tol)
    assert not bad.any(), (what, int(bad.sum()), float(err[bad].max()))


def test_tiny_workload_three_steps():
    """64x64 X and W from one generator seeded 0 (then the bias), history 4,
    three steps with X and W doubling each step, NT GEMM with bias."""
    ds = require_gpu()
    x0, w0, bias = bf16_normal_sequence([(64, 64), (64, 64), (64,)], 0)
    sx, sw = Side(ds, E4M3, 4), Side(ds, E4M3, 4)
    dbias = to_dev_bf16(bias)
    scales = []
    for t in range(3):
        dbl = lambda v: ((oracle.bf16_to_f32(v) * np.float32(2.0 ** t)).view(np.uint32) >> 16).astype(np.uint16)
        x, w = dbl(x0), dbl(w0)
        qx, cx = sx.quantize(x)
        qw, cw = sw.quantize(w)
        y = ds.fp8_mm(qx, qw, E4M3, E4M3, ds.NT, 64, 64, 64, sx.ring, sw.ring, bias=dbias)
        check_mm(ds, y, cx, cw, E4M3, E4M3, oracle.NT, 64, 64, 64, sx.s_inv, sw.s_inv, bias, what=f"step {t}")
        scales.append(sx.ref.scale)
    # closed form: after step t the published scale is s1 * 2^-t
    assert scales[1] == np.float32(scales[0] / 2) and scales[2] == np.float32(scales[0] / 4)


def test_linear_layer_dim1024_tokens2048():
    """Forward NT E4M3 with bias, then dX = G W (NN) and dW = G^T X (TN) with
    G E5M2 ~ N(0, 1e-3), backward reusing the forward's scales; two steps."""
    ds = require_gpu()
    T, D, F = 2048, 1024, 4096
    sx, sw, sg = Side(ds, E4M3, 16), Side(ds, E4M3, 16), Side(ds, E5M2, 16)
    for step in range(2):
        say(f"linear step {step}")
        x = bf16_normal((T, D), seed_for(2, step, "X"))
        w = bf16_normal((F, D), seed_for(2, step, "W"))
        bias = bf16_normal((F,), seed_for(2, step, "bias"))
        g = bf16_normal((T, F), seed_for(2, step, "G"), 1e-3)
        qx, cx = sx.quantize(x)
        qw, cw = sw.quantize(w)
        y = ds.fp8_mm(qx, qw, E4M3, E4M3, ds.NT, T, F, D, sx.ring, sw.ring, bias=to_dev_bf16(bias))
        check_mm(ds, y, cx, cw, E4M3, E4M3, oracle.NT, T, F, D, sx.s_inv, sw.s_inv, bias, what="fwd")
        qg, cg = sg.quantize(g)
        dx = ds.fp8_mm(qg, qw, E5M2, E4M3, ds.NN, T, D, F, sg.ring, sw.ring)
        check_mm(ds, dx, cg, cw, E5M2, E4M3, oracle.NN, T, D, F, sg.s_inv, sw.s_inv, what="dX")
        dw = ds.fp8_mm(qg, qx, E5M2, E4M3, ds.TN, F, D, T, sg.ring, sx.ring)
        check_mm(ds, dw, cg, cx, E5M2, E4M3, oracle.TN, F, D, T, sg.s_inv, sx.s_inv, what="dW")


def check_mm_tiles(ds, out, a_codes, b_codes, fa, fb, layout, m, n, k, sa, sb, bias=None, tile=256, what=""):
    """Compare a (single, densely stored) GPU GEMM output with the oracle on
    whole rows and whole columns: the first and the last row of every band of
    `tile` rows and the first and the last column of every band of `tile`
    columns.  Every tile x tile block of C is thus checked on two full rows
    and two full columns, its four corners included, so a tile stored to the
    wrong place or computed from the wrong operand strip cannot pass.  The
    oracle computes the selected rows (columns) as the GEMM of the matching
    rows of A (columns of B) with the whole other operand."""
    a2 = np.asarray(a_codes).reshape((k, m) if layout == oracle.TN else (m, k))
    b2 = np.asarray(b_codes).reshape((n, k) if layout == oracle.NT else (k, n))
    got = bf16_bits(out).reshape(m, n)
    amax_a = oracle.max_abs_dequant(a2, fa, sa)
    amax_b = oracle.max_abs_dequant(b2, fb, sb)

    def edges(size):
        starts = np.arange(0, size, tile)
        return np.unique(np.concatenate([starts, np.minimum(starts + tile, size) - 1]))

    rows, cols = edges(m), edges(n)
    a_rows = np.ascontiguousarray(a2[:, rows] if layout == oracle.TN else a2[rows])
    lda = len(rows) if layout == oracle.TN else k
    _, ref_r = oracle.mm(a_rows, b2, fa, fb, layout, len(rows), n, k, lda, k if layout == oracle.NT else n,
                         sa, sb, bias)
    b_cols = np.ascontiguousarray(b2[cols] if layout == oracle.NT else b2[:, cols])
    ldb = k if layout == oracle.NT else len(cols)
    _, ref_c = oracle.mm(a2, b_cols, fa, fb, layout, m, len(cols), k, m if layout == oracle.TN else k, ldb,
                         sa, sb, None if bias is None else np.asarray(bias)[cols])
    for g, r, where in ((got[rows], ref_r[0], "rows"), (got[:, cols], ref_c[0], "columns")):
        err = np.abs(oracle.bf16_to_f32(g).astype(np.float64) - oracle.bf16_to_f32(r).astype(np.float64))
        bad = ~(err <= oracle.tolerance(r, k, amax_a, amax_b))
        assert not bad.any(), (what, where, int(bad.sum()), np.argwhere(bad)[:5].tolist())


@pytest.mark.parametrize("size", [1024, 2048, 4096, 8192])
def test_square_sweep(size):
    """A, B ~ N(0,1) quantized E4M3 with 448/amax of their own tensor: the
    second delayed step applies the scale the first published.  NT, no bias."""
    ds = require_gpu()
    say(f"square {size}")
    a = bf16_normal((size, size), seed_for(3, 0, "A"))
    b = bf16_normal((size, size), seed_for(3, 0, "B"))
    sa, sb = Side(ds, E4M3, 16), Side(ds, E4M3, 16)
    full = size <= 2048
    sa.quantize(a, check_codes=full)
    sb.quantize(b, check_codes=full)
    qa, ca = sa.quantize(a)
    qb, cb = sb.quantize(b)
    assert sa.s_inv == np.float32(1.0) / (np.float32(448.0) / oracle.amax(a))
    y = ds.fp8_mm(qa, qb, E4M3, E4M3, ds.NT, size, size, size, sa.ring, sb.ring)
    if full:
        check_mm(ds, y, ca, cb, E4M3, E4M3, oracle.NT, size, size, size, sa.s_inv, sb.s_inv, what=f"square {size}")
    else:
        check_mm_tiles(ds, y, ca, cb, E4M3, E4M3, oracle.NT, size, size, size, sa.s_inv, sb.s_inv,
                       what=f"square {size}")


SKINNY = [
    ("64x8192x2048", 64, 8192, 2048, 1, False, False),
    ("1024x1536x2048", 1024, 1536, 2048, 1, False, False),
    ("1024x1000x2048 bias", 1024, 1000, 2048, 1, False, True),
    ("bmm 64 x 512^3", 512, 512, 512, 64, False, False),
    ("bmm 8 x 1024x1024x2048, B broadcast", 1024, 1024, 2048, 8, True, False),
]


@pytest.mark.parametrize("name,m,n,k,batch,bcast,with_bias", SKINNY, ids=[c[0] for c in SKINNY])
def test_skinny_and_batched(name, m, n, k, batch, bcast, with_bias):
    ds = require_gpu()
    say(name)
    a = bf16_normal((batch * m, k), seed_for(4, 0, "A"))
    b = bf16_normal(((1 if bcast else batch) * n, k), seed_for(4, 0, "B"))
    bias = bf16_normal((n,), seed_for(4, 0, "bias")) if with_bias else None
    sa, sb = Side(ds, E4M3, 16), Side(ds, E4M3, 16)
    sa.quantize(a, check_codes=False)
    sb.quantize(b, check_codes=False)
    qa, ca = sa.quantize(a)
    qb, cb = sb.quantize(b)
    y = ds.fp8_mm(qa, qb, E4M3, E4M3, ds.NT, m, n, k, sa.ring, sb.ring,
                  bias=None if bias is None else to_dev_bf16(bias), batch=batch,
                  stride_a=m * k, stride_b=0 if bcast else n * k)
    small = m * n * k * batch <= 2 ** 34
    check_mm(ds, y, ca, cb, E4M3, E4M3, oracle.NT, m, n, k, sa.s_inv, sb.s_inv, bias, batch=batch,
             stride_a=m * k, stride_b=0 if bcast else n * k, sample=None if small else 4000, what=name)
