"""Parity of the HIP scaled FP8 GEMM with the float64 oracle: every layout,
format pair and tile of the family on ragged shapes spanning several tiles,
batches with broadcast, every bias kind, exact small-integer products (bit
equality), K = 0, guard bands around the output, run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, require_gpu, say, to_dev_bf16, to_dev_u8
from synth import bf16_normal, random_codes

pytestmark = pytest.mark.gpu

FINITE = {
    oracle.E4M3: np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8),
    oracle.E5M2: np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8),
}
LAYOUTS = {"NT": oracle.NT, "NN": oracle.NN, "TN": oracle.TN}


def stored_shapes(layout, m, n, k):
    a = (k, m) if layout == oracle.TN else (m, k)
    b = (n, k) if layout == oracle.NT else (k, n)
    return a, b


def check_close(got_bits, ref_bits, k, amax_a, amax_b, what):
    got = oracle.bf16_to_f32(got_bits).astype(np.float64)
    ref = oracle.bf16_to_f32(ref_bits).astype(np.float64)
    tol = oracle.tolerance(ref_bits, k, amax_a, amax_b)
    err = np.abs(got - ref)
    bad = ~(err <= tol)
    assert not bad.any(), (what, int(bad.sum()), np.flatnonzero(bad.reshape(-1))[:5],
                           got.reshape(-1)[bad.reshape(-1)][:5], ref.reshape(-1)[bad.reshape(-1)][:5])


def scale_tensor(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda")


def run_case(ds, layout, fa, fb, m, n, k, batch=1, bcast_b=False, bias_kind=None, tile=None,
             pad_ld=0, seed=0, codes=None, sa=0.013, sb=0.021, grid=None):
    (ar, ac), (br, bc) = stored_shapes(layout, m, n, k)
    up = lambda v, q: (v + q - 1) // q * q
    lda, ldb, ldc = up(ac, 16) + pad_ld, up(bc, 16) + pad_ld, up(n, 8) + (8 if pad_ld else 0)
    stride_a, stride_b = ar * lda, (0 if bcast_b else br * ldb)
    stride_c = m * ldc
    na = stride_a * (batch - 1) + ar * lda
    nb = (stride_b * (batch - 1) if not bcast_b else 0) + br * ldb
    a = random_codes((max(na, 1),), seed + 1, FINITE[fa] if codes is None else codes)
    b = random_codes((max(nb, 1),), seed + 2, FINITE[fb] if codes is None else codes)
    bias = None
    bias_np = None
    if bias_kind is not None:
        bias_np = bf16_normal((n,), seed + 3)
        bias = to_dev_bf16(bias_np) if bias_kind == "bf16" else torch.from_numpy(oracle.bf16_to_f32(bias_np)).cuda()
    canary = 0x7FA5   # a NaN pattern no kernel produces
    out = torch.full((batch * stride_c + 64,), 0, dtype=torch.int16, device="cuda")
    out.fill_(canary - 65536 if canary > 32767 else canary)
    out = out.view(torch.bfloat16)
    ds.fp8_mm(to_dev_u8(a), to_dev_u8(b), fa, fb, layout, m, n, k, scale_tensor(sa), scale_tensor(sb),
              bias=bias, out=out, batch=batch, lda=lda, ldb=ldb, ldc=ldc, stride_a=stride_a,
              stride_b=stride_b, stride_c=stride_c, tile=tile, max_workgroups=grid)
    torch.cuda.synchronize()
    raw = bf16_bits(out)
    y, ref = oracle.mm(a, b, fa, fb, layout, m, n, k, lda, ldb, sa, sb, bias_np, batch, stride_a, stride_b)
    got = np.stack([raw[bi * stride_c: bi * stride_c + m * ldc].reshape(m, ldc)[:, :n] for bi in range(batch)])
    # guard bands: padding columns and the tail of the buffer are untouched
    full = raw[: batch * stride_c].reshape(batch, m, ldc)
    assert np.all(full[:, :, n:] == canary) and np.all(raw[batch * stride_c:] == canary)
    amax_a = oracle.max_abs_dequant(a, fa, sa)
    amax_b = oracle.max_abs_dequant(b, fb, sb)
    check_close(got, ref, k, amax_a, amax_b, (layout, fa, fb, m, n, k, batch, tile, grid))
    return got, ref


@pytest.mark.parametrize("tile", ["256x256", "128x128", "64x64", "256x128", "128x256", "256x256w8n", "256x256w8", "128x128u", "64x64u"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("fa,fb", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_layouts_formats_tiles_ragged(tile, layout, fa, fb):
    ds = require_gpu()
    say(f"gemm {layout} fmt=({fa},{fb}) tile={tile}")
    # several tiles in M and N with ragged edges, K with a ragged last stage
    run_case(ds, LAYOUTS[layout], fa, fb, 300, 520, 320, tile=tile, bias_kind="bf16", seed=7)
    # K not a multiple of 16 (zero-fixed padding), padded leading dimensions
    run_case(ds, LAYOUTS[layout], fa, fb, 130, 90, 200, tile=tile, pad_ld=16, seed=8)


@pytest.mark.parametrize("tile", ["256x256", "128x128", "64x64", "256x128", "128x256", "256x256w8n", "256x256w8", "128x128u", "64x64u"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_workgroups_running_several_tiles(tile, layout):
    """Grids of 1, 3 and 8 workgroups: each workgroup runs many output tiles
    back to back, its loads running ahead into its next tile while the
    current one computes and stores."""
    ds = require_gpu()
    say(f"gemm {layout} tile={tile} bounded grids")
    lay = LAYOUTS[layout]
    run_case(ds, lay, 1, 0, 300, 520, 320, tile=tile, bias_kind="f32", seed=30, grid=8)     # 5 stages per tile
    run_case(ds, lay, 0, 0, 130, 90, 200, tile=tile, pad_ld=16, seed=31, grid=3)           # K % 16 != 0, 4 stages
    run_case(ds, lay, 0, 1, 200, 136, 64, tile=tile, seed=32, grid=1)                      # one stage per tile
    run_case(ds, lay, 1, 1, 270, 300, 336, tile=tile, seed=34, grid=8)                     # last stage 16 of 64
    run_case(ds, lay, 0, 0, 96, 200, 128, batch=5, bcast_b=True, bias_kind="bf16", tile=tile, seed=33,
             grid=8)                                                                        # 2 stages, batches


@pytest.mark.parametrize("tile", ["256x256", "128x128", "64x64", "256x128", "128x256", "256x256w8n", "256x256w8", "128x128u", "64x64u"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_epilogue_through_lds(tile, layout):
    """No bias, so every block inside C is stored through LDS: batches, a
    padded ldc whose padding columns stay untouched, ragged edge blocks beside
    interior ones, and two workgroups running 4-5 tiles each (the staging area
    is the freed stage buffer that the next tile's loads refill)."""
    ds = require_gpu()
    say(f"gemm {layout} tile={tile} staged epilogue")
    lay = LAYOUTS[layout]
    run_case(ds, lay, 1, 0, 520, 528, 192, batch=2, tile=tile, pad_ld=16, seed=40, grid=2)
    run_case(ds, lay, 0, 0, 512, 512, 64, tile=tile, seed=41, grid=8)                      # interior only, K = 64


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_small_integer_products_bit_exact(layout):
    ds = require_gpu()
    codes = np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], np.uint8)   # 0, +-1, +-2
    for tile in ["256x256", "128x128", "64x64", "256x128", "128x256", "256x256w8n", "256x256w8", "128x128u", "64x64u"]:
        got, ref = run_case(ds, LAYOUTS[layout], 0, 0, 200, 136, 64, tile=tile, codes=codes, sa=1.0, sb=1.0, seed=3)
        assert np.array_equal(got, ref)


@pytest.mark.parametrize("bias_kind", [None, "bf16", "f32"])
def test_batches_broadcast_and_bias(bias_kind):
    ds = require_gpu()
    run_case(ds, oracle.NT, 0, 0, 96, 200, 256, batch=5, bias_kind=bias_kind, seed=11)
    run_case(ds, oracle.NT, 0, 0, 128, 136, 384, batch=4, bcast_b=True, bias_kind=bias_kind, seed=12)
    run_case(ds, oracle.NN, 1, 0, 70, 64, 130, batch=3, bias_kind=bias_kind, seed=13, tile="64x64")
    run_case(ds, oracle.TN, 1, 0, 64, 48, 520, batch=2, bcast_b=True, bias_kind=bias_kind, seed=14)


def test_k_zero_writes_bias():
    ds = require_gpu()
    for bias_kind in [None, "bf16"]:
        got, ref = run_case(ds, oracle.NT, 0, 0, 33, 47, 0, bias_kind=bias_kind, seed=15)
        assert np.array_equal(got, ref)


def test_deterministic_per_tile():
    ds = require_gpu()
    m, n, k = 512, 384, 1024
    a = to_dev_u8(random_codes((m * k,), 20, FINITE[0]))
    b = to_dev_u8(random_codes((n * k,), 21, FINITE[0]))
    for tile in ["256x256", "128x128", "64x64", "256x256w8", "128x128u", "64x64u"]:
        o1 = ds.fp8_mm(a, b, 0, 0, oracle.NT, m, n, k, scale_tensor(0.01), scale_tensor(0.01), tile=tile)
        o2 = ds.fp8_mm(a, b, 0, 0, oracle.NT, m, n, k, scale_tensor(0.01), scale_tensor(0.01), tile=tile)
        o3 = ds.fp8_mm(a, b, 0, 0, oracle.NT, m, n, k, scale_tensor(0.01), scale_tensor(0.01), tile=tile,
                       max_workgroups=3)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))   # grid size never changes the bits
