"""Parity of the widened path with the oracle: fp16 / fp32 quantize inputs,
the transposed and dual quantize (byte-equal to the row-wise codes), the
dynamic-scaling recipe, the bias-gradient column sum and the GEMM's 8-bit
bias.  Codes and ring fields bit-exact; sums within the float32 summation
bound and bit-identical run to run."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, f32_bits, require_gpu, say, to_dev_bf16, to_dev_u8
from synth import bf16_from_float, bf16_normal, random_codes
from test_gpu_quantize import assert_ring_equal

pytestmark = pytest.mark.gpu

TORCH_IN = {oracle.IN_BF16: torch.bfloat16, oracle.IN_F16: torch.float16, oracle.IN_F32: torch.float32}


def make_input(shape, seed, kind, sigma=1.0, outliers=True):
    """Seeded input bits of the given type (uint16 for bf16 / fp16, uint32 for fp32)."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32) * float(sigma)
    if outliers:
        mask = torch.rand(tuple(shape), generator=g) < 0.01
        x = torch.where(mask, x * 50.0, x)
    t = x.to(TORCH_IN[kind])
    return t.view(torch.int16 if kind != oracle.IN_F32 else torch.int32).numpy().view(
        np.uint16 if kind != oracle.IN_F32 else np.uint32)


def to_dev(bits, kind):
    arr = np.ascontiguousarray(bits)
    if kind == oracle.IN_F32:
        return torch.from_numpy(arr.view(np.int32)).view(torch.float32).cuda()
    return torch.from_numpy(arr.view(np.int16)).view(TORCH_IN[kind]).cuda()


# ---------------------------------------------------------------------------
# input types

@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp16_every_pattern(fmt):
    ds = require_gpu()
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for scale in [1.0, 448.0 / 3.25, 2.0 ** -10, 2.0 ** 12]:
        say(f"fp16 every pattern fmt={fmt} scale={scale}")
        ring = ds.ScaleRing(4, fmt, scale)
        q = ds.fp8_quantize(to_dev(h, oracle.IN_F16), fmt, ring)
        codes, ref = oracle.quantize_step(oracle.ring_init(4, fmt, scale), h, oracle.IN_F16)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), codes)
        assert_ring_equal(ring.read(), ref, scale)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_fp16_signalling_nan_is_the_amax(fmt):
    """fp16 inputs whose largest magnitude is a signalling NaN: the amax, the
    history slot and the dynamic recipe's amax keep its payload bit for bit
    (fp16 widens exactly, so 0x7C01 becomes 0x7F802000 and stays signalling);
    the codes of those elements are the NaN code with their sign.  One tensor
    per case, in the 1-D, dual and dynamic entry points."""
    ds = require_gpu()
    base = make_input((64, 96), 71, oracle.IN_F16)
    cases = [
        ("only NaN is 0x7C01", [(5, 0x7C01)]),
        ("negative sNaN 0xFD55 above a positive 0x7C01", [(7, 0xFD55), (3000, 0x7C01)]),
        ("a quiet 0x7E00 above an sNaN 0x7D00", [(11, 0x7D00), (12, 0x7E00)]),
        ("sNaN 0x7DFF above an infinity", [(100, 0x7C00), (6143, 0x7DFF)]),
    ]
    for name, planted in cases:
        x = base.copy().reshape(-1)
        for pos, bits in planted:
            x[pos] = bits
        say(f"fp16 signalling NaN fmt={fmt}: {name}")
        ring = ds.ScaleRing(4, fmt, 2.0)
        q = ds.fp8_quantize(to_dev(x, oracle.IN_F16), fmt, ring)
        codes, ref = oracle.quantize_step(oracle.ring_init(4, fmt, 2.0), x, oracle.IN_F16)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), codes), name
        assert_ring_equal(ring.read(), ref, name)
        ring2 = ds.ScaleRing(4, fmt, 2.0)
        y, y_t = ds.fp8_quantize_2d(to_dev(x.reshape(64, 96), oracle.IN_F16), fmt, ring2, oracle.DUAL)
        ry, ry_t, ref2 = oracle.quantize_step_2d(oracle.ring_init(4, fmt, 2.0), x, 64, 96, oracle.DUAL, oracle.IN_F16)
        torch.cuda.synchronize()
        assert np.array_equal(y.cpu().numpy(), ry) and np.array_equal(y_t.cpu().numpy(), ry_t), name
        assert_ring_equal(ring2.read(), ref2, name)
        check_dynamic(ds, x, oracle.IN_F16, fmt)


@pytest.mark.parametrize("kind", [oracle.IN_F16, oracle.IN_F32])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_input_types_ragged_chain(kind, fmt):
    """Five steps of mixed ragged sizes (tails shorter than one 16-byte chunk)
    through one ring, history 3."""
    ds = require_gpu()
    ring = ds.ScaleRing(3, fmt)
    ref = oracle.ring_init(3, fmt)
    for t, n in enumerate([1, 7, 4099, 100003, 3 * 1024 * 1024 + 5]):
        say(f"input type {kind} fmt={fmt} step {t} n={n}")
        x = make_input((n,), 500 + t, kind, sigma=2.0 ** (3 * t - 6))
        q = ds.fp8_quantize(to_dev(x, kind), fmt, ring)
        codes, ref = oracle.quantize_step(ref, x, kind)
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), codes), (t, n)
        assert_ring_equal(ring.read(), ref, (t, n))


# ---------------------------------------------------------------------------
# transposed / dual quantize

SHAPES_2D = [(16, 16), (48, 80), (64, 64), (144, 208), (1040, 528)]


@pytest.mark.parametrize("kind", [oracle.IN_BF16, oracle.IN_F16, oracle.IN_F32])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_orientations_match_oracle_and_rowwise(kind, fmt):
    ds = require_gpu()
    for rows, cols in SHAPES_2D:
        say(f"2-D quantize kind={kind} fmt={fmt} {rows}x{cols}")
        x = make_input((rows, cols), rows * 7 + cols, kind, sigma=3.0)
        xd = to_dev(x, kind)
        outs = {}
        for layout in [oracle.ROWWISE, oracle.TRANSPOSED, oracle.DUAL]:
            ring = ds.ScaleRing(2, fmt, 0.75)
            y, y_t = ds.fp8_quantize_2d(xd, fmt, ring, layout)
            ry, ry_t, rring = oracle.quantize_step_2d(oracle.ring_init(2, fmt, 0.75), x, rows, cols, layout, kind)
            torch.cuda.synchronize()
            if ry is not None:
                assert np.array_equal(y.cpu().numpy(), ry), (layout, rows, cols)
            if ry_t is not None:
                assert np.array_equal(y_t.cpu().numpy(), ry_t), (layout, rows, cols)
            assert_ring_equal(ring.read(), rring, (layout, rows, cols))
            outs[layout] = (y, y_t)
        # byte equality between the GPU's own orientations
        row = outs[oracle.ROWWISE][0]
        assert torch.equal(outs[oracle.TRANSPOSED][1], row.t().contiguous())
        assert torch.equal(outs[oracle.DUAL][0], row) and torch.equal(outs[oracle.DUAL][1], row.t().contiguous())


def test_dual_at_linear_shapes_with_nan_inf():
    """The linear layer's X [4096, 1024] and G [4096, 4096] at full size, one
    NaN and one inf planted, over a 3-step ring."""
    ds = require_gpu()
    for shape, fmt in [((4096, 1024), oracle.E4M3), ((4096, 4096), oracle.E5M2)]:
        ring = ds.ScaleRing(16, fmt)
        ref = oracle.ring_init(16, fmt)
        for t in range(3):
            say(f"dual {shape} step {t}")
            x = bf16_normal(shape, 900 + t, 1e-3 if fmt == oracle.E5M2 else 1.0, outliers=True)
            if t == 2:
                x = x.copy()
                x[5, 7] = 0xFFC1      # NaN with the sign bit set
                x[100, 3] = 0x7F80    # +inf
            y, y_t = ds.fp8_quantize_2d(to_dev_bf16(x), fmt, ring, oracle.DUAL)
            ry, ry_t, ref = oracle.quantize_step_2d(ref, x, shape[0], shape[1], oracle.DUAL)
            torch.cuda.synchronize()
            assert np.array_equal(y.cpu().numpy(), ry) and np.array_equal(y_t.cpu().numpy(), ry_t), (shape, t)
            assert_ring_equal(ring.read(), ref, (shape, t))


# ---------------------------------------------------------------------------
# dynamic recipe

def check_dynamic(ds, x, kind, fmt):
    ring = ds.ScaleRing(1, fmt, 3.0)          # its initial scale must not matter
    q = ds.fp8_quantize_dynamic(to_dev(x, kind), fmt, ring)
    codes, s, s_inv, a = oracle.quantize_dynamic(x, fmt, kind)
    want = oracle.dynamic_ring_after(x, fmt, kind)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), codes)
    assert_ring_equal(ring.read(), want, (kind, fmt, x.size))


@pytest.mark.parametrize("kind", [oracle.IN_BF16, oracle.IN_F16, oracle.IN_F32])
@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_dynamic_matches_oracle(kind, fmt):
    ds = require_gpu()
    for n, sigma in [(1, 1.0), (4101, 1e-3), (2 * 1024 * 1024 + 3, 40.0)]:
        say(f"dynamic kind={kind} fmt={fmt} n={n}")
        check_dynamic(ds, make_input((n,), n + 17, kind, sigma), kind, fmt)


def test_dynamic_degenerate_tensors():
    ds = require_gpu()
    for vals in ([0.0] * 9, [1.0, np.inf, 2.0], [1.0, np.nan, -3.0], [2.0 ** -130, 0.0]):
        check_dynamic(ds, bf16_from_float(np.array(vals, np.float32)), oracle.IN_BF16, oracle.E4M3)


# ---------------------------------------------------------------------------
# bias gradient

def check_bias_grad(ds, g_np, rows, cols, kind, fmt=None, s_inv=None, out_f32=False, ws=None):
    if kind is None:
        g = to_dev_u8(g_np.reshape(rows, cols))
        sd = torch.tensor([s_inv], dtype=torch.float32, device="cuda")
        out = ds.fp8_bias_grad(g, rows, cols, fmt=fmt, g_scale_inv=sd, out_f32=out_f32, workspace=ws)
    else:
        g = to_dev(g_np.reshape(rows, cols), kind)
        out = ds.fp8_bias_grad(g, rows, cols, out_f32=out_f32, workspace=ws)
    exact, bits, f = oracle.bias_grad(g_np, rows, cols, kind, fmt, s_inv)
    torch.cuda.synchronize()
    if out_f32:
        got, ref, ok = out.cpu().numpy().astype(np.float64), f.astype(np.float64), oracle.OUT_F32
        tol = oracle.bias_grad_tolerance(g_np, rows, cols, kind, f, ok, fmt, s_inv)
    else:
        got, ref = oracle.bf16_to_f32(bf16_bits(out)).astype(np.float64), oracle.bf16_to_f32(bits).astype(np.float64)
        tol = oracle.bias_grad_tolerance(g_np, rows, cols, kind, bits, oracle.OUT_BF16, fmt, s_inv)
    bad = ~(np.abs(got - ref) <= tol)
    assert not bad.any(), (rows, cols, kind, np.flatnonzero(bad)[:5], got[bad][:5], ref[bad][:5])
    return out


@pytest.mark.parametrize("kind", [oracle.IN_BF16, oracle.IN_F16, oracle.IN_F32])
def test_bias_grad_types_and_shapes(kind):
    ds = require_gpu()
    for rows, cols in [(0, 8), (1, 8), (33, 72), (2048, 4096), (4096, 1024), (777, 136)]:
        for out_f32 in (False, True):
            say(f"bias grad kind={kind} {rows}x{cols} out_f32={out_f32}")
            g = make_input((rows, cols), rows + cols, kind, sigma=1e-3, outliers=True)
            check_bias_grad(ds, g, rows, cols, kind, out_f32=out_f32)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_bias_grad_of_codes(fmt):
    ds = require_gpu()
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F and (fmt == oracle.E4M3 or (c & 0x7C) != 0x7C)],
                      np.uint8)
    for rows, cols in [(5, 16), (2048, 4096)]:
        say(f"bias grad codes fmt={fmt} {rows}x{cols}")
        codes = random_codes((rows * cols,), rows + 1, finite)
        check_bias_grad(ds, codes, rows, cols, None, fmt, np.float32(3.0e-4))


def test_bias_grad_deterministic_and_workspace_reuse():
    ds = require_gpu()
    rows, cols = 3000, 1032
    ws = ds.BiasGradWorkspace(rows, cols)
    g = make_input((rows, cols), 77, oracle.IN_BF16, sigma=1.0)
    first = check_bias_grad(ds, g, rows, cols, oracle.IN_BF16, out_f32=True, ws=ws)
    again = check_bias_grad(ds, g, rows, cols, oracle.IN_BF16, out_f32=True, ws=ws)
    assert torch.equal(first.view(torch.int32), again.view(torch.int32))
    torch.cuda.synchronize()
    assert int(ws.buf.sum()) == 0                          # every call leaves the workspace zero
    # so it serves calls of other shapes it covers
    check_bias_grad(ds, make_input((64, 64), 78, oracle.IN_BF16), 64, 64, oracle.IN_BF16, ws=ws)
    check_bias_grad(ds, make_input((3000, 1032), 79, oracle.IN_F16), 3000, 1032, oracle.IN_F16, ws=ws)
    torch.cuda.synchronize()
    assert int(ws.buf.sum()) == 0


# ---------------------------------------------------------------------------
# GEMM with an 8-bit bias

@pytest.mark.parametrize("bfmt", [oracle.E4M3, oracle.E5M2])
@pytest.mark.parametrize("layout", [oracle.NT, oracle.NN, oracle.TN])
def test_gemm_fp8_bias(bfmt, layout):
    ds = require_gpu()
    m, n, k = 300, 1000, 256
    (ar, ac) = (k, m) if layout == oracle.TN else (m, k)
    (br, bc) = (n, k) if layout == oracle.NT else (k, n)
    fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    lda, ldb = (ac + 15) // 16 * 16, (bc + 15) // 16 * 16      # leading dimensions padded to 16 bytes
    a = random_codes((ar * lda,), 61, fin)
    b = random_codes((br * ldb,), 62, fin)
    fin_b = np.array([c for c in range(256) if (c & 0x7F) < 0x70], np.uint8)
    bias = random_codes((n,), 63, fin_b)
    bsi = np.float32(0.37)
    sa, sb = 0.011, 0.017
    out = ds.fp8_mm(to_dev_u8(a), to_dev_u8(b), 0, 0, layout, m, n, k,
                    torch.tensor([sa], dtype=torch.float32, device="cuda"),
                    torch.tensor([sb], dtype=torch.float32, device="cuda"),
                    bias=to_dev_u8(bias), bias_fmt=bfmt, lda=lda, ldb=ldb,
                    bias_scale_inv=torch.tensor([bsi], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    y, ref = oracle.mm(a, b, 0, 0, layout, m, n, k, lda, ldb, sa, sb, bias=bias, bias_fmt=bfmt, bias_scale_inv=bsi)
    got = oracle.bf16_to_f32(bf16_bits(out).reshape(m, n)).astype(np.float64)
    r = oracle.bf16_to_f32(ref[0]).astype(np.float64)
    tol = oracle.tolerance(ref[0], k, oracle.max_abs_dequant(a, 0, sa), oracle.max_abs_dequant(b, 0, sb))
    assert np.all(np.abs(got - r) <= tol)
