"""The bias gradient's no-allocation entry point (fp8_bias_grad_noalloc, its
scratch in the library's own device array) against the workspace entry point
it varies (fp8_bias_grad): the same bits for the same input, on calls in a row
whose second is smaller than the first, so the shared scratch must come back
clean from each call; both within the oracle's summation bound.  Shapes past
the array's size are refused."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, require_gpu, say, to_dev_bf16, to_dev_u8
from synth import bf16_normal, random_codes

pytestmark = pytest.mark.gpu


def check_against_workspace_entry(ds, g_dev, g_np, rows, cols, kind, fmt=None, s_inv=None, out_f32=False):
    odt = torch.float32 if out_f32 else torch.bfloat16
    out_na = torch.full((cols,), 7.0, dtype=odt, device="cuda")
    kw = {} if fmt is None else dict(fmt=fmt, g_scale_inv=torch.tensor([s_inv], dtype=torch.float32, device="cuda"))
    ds.fp8_bias_grad_noalloc(g_dev, rows, cols, out_f32=out_f32, out=out_na, **kw)
    ws = ds.BiasGradWorkspace(rows, cols)
    out_ws = ds.fp8_bias_grad(g_dev, rows, cols, out_f32=out_f32, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out_na.view(torch.int32 if out_f32 else torch.int16),
                       out_ws.view(torch.int32 if out_f32 else torch.int16)), (rows, cols, kind, fmt)
    exact, bits, f = oracle.bias_grad(g_np, rows, cols, kind, fmt, s_inv)
    if out_f32:
        got = out_na.cpu().numpy().astype(np.float64)
        tol = oracle.bias_grad_tolerance(g_np, rows, cols, kind, f, oracle.OUT_F32, fmt, s_inv)
        ref = f.astype(np.float64)
    else:
        got = oracle.bf16_to_f32(bf16_bits(out_na)).astype(np.float64)
        tol = oracle.bias_grad_tolerance(g_np, rows, cols, kind, bits, oracle.OUT_BF16, fmt, s_inv)
        ref = oracle.bf16_to_f32(bits).astype(np.float64)
    assert np.all(np.abs(got - ref) <= tol), (rows, cols)


def test_noalloc_matches_workspace_entry_two_calls_second_smaller():
    ds = require_gpu()
    for rows, cols in [(4096, 4096), (2048, 1024), (37, 24), (256, 65536), (1, 8)]:
        say(f"noalloc bias grad bf16 {rows}x{cols}")
        g = bf16_normal((rows, cols), rows * 31 + cols, 1e-3, outliers=True)
        check_against_workspace_entry(ds, to_dev_bf16(g), g, rows, cols, oracle.IN_BF16)
    for out_f32 in (True, False):
        say(f"noalloc bias grad of E5M2 codes, out_f32={out_f32}")
        for rows, cols in [(3000, 2048), (100, 512)]:
            codes = random_codes((rows, cols), rows + cols, np.array(
                [c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8))
            check_against_workspace_entry(ds, to_dev_u8(codes), codes, rows, cols, None, oracle.E5M2,
                                          np.float32(2.0 ** -7), out_f32)


def test_noalloc_refuses_shapes_past_its_scratch():
    ds = require_gpu()
    cols = 1 << 19                                   # one slice of 2^19 fp32 partials: 2 MiB
    assert ds.bias_grad_workspace_bytes(64, cols) > ds.NOALLOC_MAX_BYTES
    g = torch.zeros((64, cols), dtype=torch.bfloat16, device="cuda")
    out = torch.empty(cols, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ds.Fp8dsError, match="scratch"):
        ds.fp8_bias_grad_noalloc(g, out=out)
    # and the entry point still works afterwards
    g2 = bf16_normal((128, 256), 5, 1.0)
    check_against_workspace_entry(ds, to_dev_bf16(g2), g2, 128, 256, oracle.IN_BF16)
