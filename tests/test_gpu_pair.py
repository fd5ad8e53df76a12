"""The GEMM pair (a layer's dX and dW in one launch): each output is the bits
of its own fp8_mm call, both follow the oracle within the GEMM tolerance, on
ragged shapes, on pairs larger than the device holds at once (the workgroups
split between the problems and run several tiles each), with a bias, with an
empty problem, and for pairs that run as two launches."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import bf16_bits, require_gpu, say, to_dev_u8
from synth import bf16_normal, random_codes
from test_gpu_gemm import FINITE, check_close, scale_tensor, stored_shapes

pytestmark = pytest.mark.gpu


def problem(layout, fa, fb, m, n, k, seed, sa, sb, bias=False):
    """Dense operands of one GEMM on both sides, as fp8_mm keyword arguments."""
    (ar, ac), (br, bc) = stored_shapes(layout, m, n, k)
    a = random_codes((ar, ac), seed + 1, FINITE[fa])
    b = random_codes((br, bc), seed + 2, FINITE[fb])
    bias_np = bf16_normal((n,), seed + 3) if bias else None
    kw = dict(a=to_dev_u8(a), b=to_dev_u8(b), fmt_a=fa, fmt_b=fb, layout=layout, m=m, n=n, k=k,
              a_scale_inv=scale_tensor(sa), b_scale_inv=scale_tensor(sb))
    if bias:
        kw["bias"] = torch.from_numpy(bias_np.view(np.int16)).view(torch.bfloat16).cuda()
    return kw, (a, b, bias_np)


def oracle_check(out, host, kw, sa, sb, what):
    a, b, bias_np = host
    m, n, k, layout, fa, fb = kw["m"], kw["n"], kw["k"], kw["layout"], kw["fmt_a"], kw["fmt_b"]
    (_, ac), (_, bc) = stored_shapes(layout, m, n, k)
    y, ref = oracle.mm(a.reshape(-1), b.reshape(-1), fa, fb, layout, m, n, k, ac, bc, sa, sb, bias_np)
    got = bf16_bits(out).reshape(m, n)[None]
    check_close(got, ref, k, oracle.max_abs_dequant(a, fa, sa), oracle.max_abs_dequant(b, fb, sb), what)


def same_bits(p, q):
    return torch.equal(p.reshape(-1).view(torch.int16), q.reshape(-1).view(torch.int16))


@pytest.mark.parametrize("fa,fb", [(1, 0), (0, 0), (1, 1)])
def test_pair_ragged_matches_oracle_and_single_calls(fa, fb):
    """dX = G.W (NN) and dW = G^T.X (TN) of a layer with ragged sizes."""
    ds = require_gpu()
    t, n_in, n_out = 304, 208, 144      # ragged against every tile, leading dimensions multiples of 16
    sa, sb, sc = 0.0173, 0.0219, 0.0311
    dx, hx = problem(oracle.NN, fa, fb, t, n_in, n_out, 10, sa, sb, bias=True)
    dw, hw = problem(oracle.TN, fa, fb, n_out, n_in, t, 20, sa, sc)
    say(f"pair ragged fa={fa} fb={fb}")
    o0, o1 = ds.fp8_mm_pair(dx, dw)
    s0, s1 = ds.fp8_mm(**dx), ds.fp8_mm(**dw)
    torch.cuda.synchronize()
    assert same_bits(o0, s0) and same_bits(o1, s1)
    oracle_check(o0, hx, dx, sa, sb, "dX")
    oracle_check(o1, hw, dw, sa, sc, "dW")


@pytest.mark.parametrize("t,n_in,n_out", [(2048, 1024, 3072), (2048, 1024, 1024), (2048, 4096, 1024),
                                          (4096, 4096, 1024), (4096, 4096, 4096), (11264, 1024, 11264)])
def test_pair_at_layer_shapes_equals_single_calls(t, n_in, n_out):
    """The linear layer's backward shapes, plus sampled entries against the
    oracle.  At 4096 x 4096 x 1024 the pair runs as one launch on the 128x128
    unit tile with 1280 tiles, more than the device holds at once, so its
    workgroups run several tiles each; at 4096 x 4096 x 4096 and at 11264 the
    rule's tile for the pair is the eight-wave 256x256 one, so the two go out
    as separate launches."""
    ds = require_gpu()
    sa, sb, sc = 0.011, 0.017, 0.023
    dx, hx = problem(oracle.NN, 1, 0, t, n_in, n_out, 30, sa, sb)
    dw, hw = problem(oracle.TN, 1, 0, n_out, n_in, t, 40, sa, sc)
    say(f"pair {t}x{n_in}x{n_out}")
    o0, o1 = ds.fp8_mm_pair(dx, dw)
    s0, s1 = ds.fp8_mm(**dx), ds.fp8_mm(**dw)
    torch.cuda.synchronize()
    assert same_bits(o0, s0) and same_bits(o1, s1)
    rng = np.random.default_rng(t + n_in + n_out)
    for out, host, kw, s2 in ((o0, hx, dx, sb), (o1, hw, dw, sc)):
        a, b, _ = host
        m, n, k, layout = kw["m"], kw["n"], kw["k"], kw["layout"]
        (_, ac), (_, bc) = stored_shapes(layout, m, n, k)
        rows = rng.integers(0, m, 64)
        cols = rng.integers(0, n, 64)
        _, ref = oracle.mm_entries(a.reshape(-1), b.reshape(-1), 1, 0, layout, m, n, k, ac, bc, sa, s2,
                                   np.zeros(64, np.int64), rows, cols)
        got = bf16_bits(out).reshape(m, n)[rows, cols]
        check_close(got, ref, k, oracle.max_abs_dequant(a, 1, sa), oracle.max_abs_dequant(b, 0, s2), (m, n, k))


def test_pair_other_layouts_and_empty_problems():
    """A pair that is not NN + TN runs as two launches; an empty problem is
    skipped and the other still runs."""
    ds = require_gpu()
    p0, _ = problem(oracle.NT, 0, 0, 160, 96, 128, 50, 0.5, 0.25)
    p1, _ = problem(oracle.NT, 0, 0, 64, 48, 80, 60, 0.125, 0.5)
    o0, o1 = ds.fp8_mm_pair(p0, p1)
    s0, s1 = ds.fp8_mm(**p0), ds.fp8_mm(**p1)
    empty, _ = problem(oracle.NN, 1, 0, 0, 32, 64, 70, 1.0, 1.0)
    q0, q1 = ds.fp8_mm_pair(empty, p1)
    torch.cuda.synchronize()
    assert same_bits(o0, s0) and same_bits(o1, s1) and same_bits(q1, s1) and q0.numel() == 0


def test_results_do_not_depend_on_the_tile():
    """The pair may pick another tile than a single call: every tile gives the
    same bits on non-integer data (the K sum runs in one order per element)."""
    ds = require_gpu()
    for layout in (oracle.NT, oracle.NN, oracle.TN):
        kw, _ = problem(layout, 1, 0, 320, 288, 448, 80 + layout, 0.0137, 0.0291, bias=True)
        outs = [ds.fp8_mm(**kw, tile=t) for t in range(len(ds.TILES))]
        torch.cuda.synchronize()
        for t in range(1, len(outs)):
            assert same_bits(outs[0], outs[t]), (layout, t)


def test_pair_of_batched_problems():
    """Batched NN and TN problems (strided batches, and a weight broadcast with
    batch stride 0 in the first) in one pair launch equal their single calls."""
    ds = require_gpu()
    batch, t, n_in, n_out = 3, 272, 160, 208
    rng_codes = lambda shape, seed, fmt: to_dev_u8(random_codes(shape, seed, FINITE[fmt]))
    g8 = rng_codes((batch, t, n_out), 90, 1)
    w8 = rng_codes((n_out, n_in), 91, 0)                      # shared by every batch entry
    x8 = rng_codes((batch, t, n_in), 92, 0)
    s = [scale_tensor(v) for v in (0.013, 0.029, 0.041)]
    dx = dict(a=g8, b=w8, fmt_a=1, fmt_b=0, layout=oracle.NN, m=t, n=n_in, k=n_out, a_scale_inv=s[0],
              b_scale_inv=s[1], batch=batch, stride_a=t * n_out, stride_b=0, stride_c=t * n_in)
    dw = dict(a=g8, b=x8, fmt_a=1, fmt_b=0, layout=oracle.TN, m=n_out, n=n_in, k=t, a_scale_inv=s[0],
              b_scale_inv=s[2], batch=batch, stride_a=t * n_out, stride_b=t * n_in, stride_c=n_out * n_in)
    o0, o1 = ds.fp8_mm_pair(dx, dw)
    s0, s1 = ds.fp8_mm(**dx), ds.fp8_mm(**dw)
    torch.cuda.synchronize()
    assert same_bits(o0, s0) and same_bits(o1, s1)
