"""The C ABI library loads on the host and exports every function that
include/fp8ds.h declares; argument checks that return before any HIP call
report the documented status codes.  CPU only: no kernel is launched."""
import ctypes
import os
import re

import pytest

import delayed_scaling_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ds.LIB_PATH):
        pytest.fail("libfp8ds.so is not built (run __graft_entry__.build())")
    return ds.lib()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["fp8_quantize", "fp8_mm", "scale_ring_init", "fp8_scale_ring_bytes", "fp8_last_error"]:
        assert required in names


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_ring_bytes(L):
    assert ds.scale_ring_bytes(0) == 0
    assert ds.scale_ring_bytes(1025) == 0
    assert ds.scale_ring_bytes(1) == 2112 + 16
    assert ds.scale_ring_bytes(4) == 2112 + 16
    assert ds.scale_ring_bytes(16) == 2112 + 64
    assert ds.scale_ring_bytes(1024) == 2112 + 4096
    assert L.fp8_ring_scale_inv(ctypes.c_void_p(4096)) == 4100


def test_validation_errors_launch_nothing(L):
    # each of these returns before touching the GPU
    assert L.fp8_quantize(None, 16, 7, ctypes.c_void_p(64), None, None) == -1
    assert b"fmt" in L.fp8_last_error()
    assert L.fp8_quantize(None, -1, 0, ctypes.c_void_p(64), None, None) == -1
    assert L.fp8_quantize(None, 16, 0, None, None, None) == -3
    assert L.fp8_quantize(None, 16, 0, ctypes.c_void_p(65), None, None) == -2
    assert L.fp8_quantize(None, 0, 0, ctypes.c_void_p(64), None, None) == 0      # empty: no-op
    assert L.scale_ring_init(None, 4, 0, 1.0, None) == -1
    assert L.scale_ring_init(ctypes.c_void_p(64), 0, 0, 1.0, None) == -1
    assert L.scale_ring_init(ctypes.c_void_p(64), 4, 0, 0.0, None) == -1
    assert L.scale_ring_init(ctypes.c_void_p(64), 4, 0, float("inf"), None) == -1
    assert L.scale_ring_init(ctypes.c_void_p(72), 4, 0, 1.0, None) == -2
    args = ds._MmArgs()
    args.layout = 5
    assert L.fp8_mm(ctypes.byref(args), None) == -1
    assert b"layout" in L.fp8_last_error()
    args.layout = 0
    args.m, args.n, args.k = 0, 16, 16
    assert L.fp8_mm(ctypes.byref(args), None) == 0                                # empty: no-op
    args.m = 16
    assert L.fp8_mm(ctypes.byref(args), None) == -1                               # null pointers
    args.a, args.b, args.c = 4096, 8192, 16384
    args.a_scale_inv, args.b_scale_inv = 32768, 32768
    args.lda, args.ldb, args.ldc = 8, 16, 16                                      # lda < K
    assert L.fp8_mm(ctypes.byref(args), None) == -1
    args.lda = 24                                                                 # not a multiple of 16
    assert L.fp8_mm(ctypes.byref(args), None) == -2
    args.lda = 16
    args.a = 4100                                                                 # misaligned base
    assert L.fp8_mm(ctypes.byref(args), None) == -2
    args.a = 4096
    args.bias_kind = 1                                                            # bias kind without pointer
    assert L.fp8_mm(ctypes.byref(args), None) == -1
    args.bias_kind = 0
    assert L.fp8_mm_with_grid(ctypes.byref(args), -1, -1, None) == -1             # negative grid bound
    assert b"max_workgroups" in L.fp8_last_error()
    args.m = 1 << 31
    assert L.fp8_mm(ctypes.byref(args), None) == -1
    args.m, args.k, args.lda, args.ldb = 1 << 20, 1 << 12, 1 << 12, 1 << 12       # 4 GiB operand
    assert L.fp8_mm(ctypes.byref(args), None) == -3


def test_widened_entry_points_validate_before_launch(L):
    v = ctypes.c_void_p
    ring = v(4096)
    # bad input type / layout / misaligned transposed shapes
    assert L.fp8_quantize_ex(v(64), 16, 7, 0, ring, v(128), None) == -1
    assert b"in_type" in L.fp8_last_error()
    assert L.fp8_quantize_ex(v(64), 0, 2, 0, ring, v(128), None) == 0             # empty: no-op
    assert L.fp8_quantize_2d(v(64), 16, 16, 0, 0, 9, ring, v(128), v(256), None) == -1
    x, yt = v(1 << 20), v(1 << 24)
    assert L.fp8_quantize_2d(x, 24, 16, 0, 0, 1, ring, None, yt, None) == -2
    assert L.fp8_quantize_2d(x, 16, 16, 0, 0, 2, ring, None, yt, None) == -1          # DUAL without y
    assert L.fp8_quantize_2d(v(64), 0, 16, 0, 0, 2, ring, None, None, None) == 0       # empty: no-op
    assert L.fp8_quantize_dynamic(v(64), 16, 0, 0, None, v(128), None) == -3
    # bias gradient
    assert L.fp8_bias_grad_workspace_bytes(2048, 4096) > 0
    assert L.fp8_bias_grad_workspace_bytes(-1, 8) == 0
    assert L.fp8_bias_grad(v(64), 16, 12, 0, None, 0, v(128), v(256), None) == -2      # cols % 8
    assert L.fp8_bias_grad(v(64), 16, 16, 3, None, 0, v(128), v(256), None) == -1      # codes need a scale
    assert L.fp8_bias_grad(v(64), 16, 16, 9, None, 0, v(128), v(256), None) == -1
    assert L.fp8_bias_grad(v(64), 16, 0, 0, None, 0, None, None, None) == 0            # no columns: no-op
    # GEMM 8-bit bias needs its scale
    args = ds._MmArgs()
    args.m, args.n, args.k = 16, 16, 16
    args.a, args.b, args.c = 4096, 8192, 16384
    args.a_scale_inv, args.b_scale_inv = 32768, 32768
    args.lda, args.ldb, args.ldc = 16, 16, 16
    args.bias, args.bias_kind = 40960, 3
    assert L.fp8_mm(ctypes.byref(args), None) == -1
    assert b"bias_scale_inv" in L.fp8_last_error()
    args.bias_kind = 5
    assert L.fp8_mm(ctypes.byref(args), None) == -1


def test_batch_quantize_validates_before_launch(L):
    v = ctypes.c_void_p
    J = ds._QuantJob

    def jobs(*js):
        arr = (J * max(1, len(js)))()
        for i, j in enumerate(js):
            arr[i] = J(*j)
        return arr

    a = (1 << 20, 4096, 1 << 12, 1 << 24, None)          # x, numel, ring, y, scale_inv_out
    b = (1 << 21, 4096, 1 << 13, 1 << 25, None)
    assert L.fp8_quantize_batch(None, 1, 0, 0, None) == -1
    assert L.fp8_quantize_batch(jobs(a), 0, 0, 0, None) == -1
    assert L.fp8_quantize_batch(jobs(*([a] * 9)), 9, 0, 0, None) == -1
    assert b"njobs" in L.fp8_last_error()
    assert L.fp8_quantize_batch(jobs(a, b), 2, 3, 0, None) == -1                    # in_type
    assert L.fp8_quantize_batch(jobs(a, b), 2, 0, 2, None) == -1                    # fmt
    shared = (1 << 21, 4096, 1 << 12, 1 << 25, None)
    assert L.fp8_quantize_batch(jobs(a, shared), 2, 0, 0, None) == -1
    assert b"share a ring" in L.fp8_last_error()
    y_on_x = (1 << 21, 4096, 1 << 13, 1 << 20, None)                                # b's y is a's x
    assert L.fp8_quantize_batch(jobs(a, y_on_x), 2, 0, 0, None) == -1
    assert b"overlaps" in L.fp8_last_error()
    assert L.fp8_quantize_batch(jobs(a, (1 << 21, 4096, 1 << 13, 1 << 24, None)), 2, 0, 0, None) == -1   # same y
    assert L.fp8_quantize_batch(jobs(a, (1 << 21, 4096, 1 << 13, 1 << 25, 1 << 26 | 2)), 2, 0, 0, None) == -2
    assert L.fp8_quantize_batch(jobs((1 << 21, 4096, None, 1 << 25, None)), 1, 0, 0, None) == -3   # no ring
    assert L.fp8_quantize_batch(jobs((1 << 21 | 8, 4096, 1 << 13, 1 << 25, None)), 1, 0, 0, None) == -2
    empty = (None, 0, 1 << 14, None, None)
    assert L.fp8_quantize_batch(jobs(empty, empty[:2] + (1 << 15,) + empty[3:]), 2, 0, 0, None) == 0   # nothing to do


def test_mm_pair_validates_before_launch(L):
    def args(a, b, c, layout=1, m=16, n=16, k=16):
        x = ds._MmArgs()
        x.a, x.b, x.c, x.layout, x.m, x.n, x.k = a, b, c, layout, m, n, k
        x.a_scale_inv, x.b_scale_inv = 1 << 30, 1 << 30
        x.lda = x.ldb = x.ldc = 16
        return x
    first = args(1 << 20, 1 << 21, 1 << 22)
    second = args(1 << 23, 1 << 24, 1 << 25, layout=2)
    assert L.fp8_mm_pair(None, ctypes.byref(second), None) == -1
    bad = args(1 << 23, 1 << 24, 1 << 25, layout=7)
    assert L.fp8_mm_pair(ctypes.byref(first), ctypes.byref(bad), None) == -1
    onto_a = args(1 << 23, 1 << 24, 1 << 20, layout=2)          # second writes first's A
    assert L.fp8_mm_pair(ctypes.byref(first), ctypes.byref(onto_a), None) == -1
    assert b"overlaps" in L.fp8_last_error()
    same_c = args(1 << 23, 1 << 24, (1 << 22) + 256, layout=2)   # outputs overlap
    assert L.fp8_mm_pair(ctypes.byref(first), ctypes.byref(same_c), None) == -1
    e0, e1 = args(None, None, 1 << 22, m=0), args(None, None, 1 << 25, n=0, layout=2)
    assert L.fp8_mm_pair(ctypes.byref(e0), ctypes.byref(e1), None) == 0       # both empty: nothing to do


def test_mm_rejects_output_overlapping_an_input(L):
    """fp8_mm's output may not share bytes with A, B or the bias (each is
    still read while C is written); the check runs before any launch."""
    def args(c, bias=None):
        x = ds._MmArgs()
        x.m, x.n, x.k = 64, 64, 64
        x.a, x.b, x.c = 1 << 20, 1 << 21, c
        x.a_scale_inv, x.b_scale_inv = 1 << 30, 1 << 30
        x.lda = x.ldb = x.ldc = 64
        if bias is not None:
            x.bias, x.bias_kind = bias, 1
        return x
    for c in [(1 << 20) + 4096 - 16, (1 << 20) - 64 * 64 * 2 + 16, (1 << 21) + 2048]:   # ends in A, starts in A, in B
        assert L.fp8_mm(ctypes.byref(args(c)), None) == -1, hex(c)
        assert b"overlaps" in L.fp8_last_error()
    bias = (1 << 22) + 100 * 16
    assert L.fp8_mm(ctypes.byref(args(1 << 22, bias)), None) == -1                  # c covers the bias
    assert b"overlaps" in L.fp8_last_error()
    # batched: the second output entry lands on A
    x = args((1 << 20) - 2 * 64 * 64 * 2 + 16)
    x.batch, x.stride_a, x.stride_b, x.stride_c = 2, 64 * 64, 64 * 64, 64 * 64
    assert L.fp8_mm(ctypes.byref(x), None) == -1


def test_binding_checks_tensors_before_the_call():
    """The binding refuses a tensor of the wrong dtype, a non-contiguous one, a
    buffer shorter than the extent the kernel touches, and host memory, before
    anything reaches the library (CPU tensors stand in for device ones)."""
    import torch
    u8 = lambda n: torch.zeros(n, dtype=torch.uint8)
    with pytest.raises(ds.Fp8dsError, match="dtype"):
        ds._need(torch.zeros(4, dtype=torch.int16), "a", ds._U8, 4)
    with pytest.raises(ds.Fp8dsError, match="contiguous"):
        ds._need(u8(64).view(8, 8).t(), "a", ds._U8, 8)
    with pytest.raises(ds.Fp8dsError, match="holds 63 bytes"):
        ds._need(u8(63), "a", ds._U8, 64)
    with pytest.raises(ds.Fp8dsError, match="device tensor"):
        ds._need(u8(64), "a", ds._U8, 64)
    with pytest.raises(ds.Fp8dsError, match="is required"):
        ds._need(None, "a", ds._U8, 64)
    # fp8_mm's extents: NT 64 x 96 x 128 needs A 64*128, B 96*128, C 64*96 bf16
    a, b = u8(64 * 128), u8(96 * 128)
    out = torch.empty(64 * 96, dtype=torch.bfloat16)
    with pytest.raises(ds.Fp8dsError, match="out holds"):
        ds.fp8_mm(a, b, 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, out=out[:-1])
    with pytest.raises(ds.Fp8dsError, match="^a holds"):
        ds.fp8_mm(a[:-1], b, 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, out=out)
    with pytest.raises(ds.Fp8dsError, match="^b holds"):
        ds.fp8_mm(a, b[:-16], 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, out=out)
    with pytest.raises(ds.Fp8dsError, match="out has dtype"):
        ds.fp8_mm(a, b, 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, out=out.float())
    # a padded leading dimension and a batch stride count in the extent
    with pytest.raises(ds.Fp8dsError, match="^a holds"):
        ds.fp8_mm(u8(63 * 144 + 127), b, 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, lda=144, out=out)
    with pytest.raises(ds.Fp8dsError, match="out holds"):
        ds.fp8_mm(u8(2 * 64 * 128), u8(2 * 96 * 128), 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30,
                  batch=2, out=out)
    with pytest.raises(ds.Fp8dsError, match="bias holds"):
        ds.fp8_mm(a, b, 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, out=out,
                  bias=torch.zeros(95, dtype=torch.bfloat16))
    with pytest.raises(ds.Fp8dsError, match="a_scale_inv has dtype"):
        ds.fp8_mm(a, b, 0, 0, ds.NT, 64, 96, 128, torch.zeros(1, dtype=torch.float64), 1 << 30, out=out)
    with pytest.raises(ds.Fp8dsError, match="device tensor"):       # right sizes, host memory
        ds.fp8_mm(a, b, 0, 0, ds.NT, 64, 96, 128, 1 << 30, 1 << 30, out=out)
    # the bias gradient's output and workspace
    g = torch.zeros(32, 64, dtype=torch.bfloat16)
    with pytest.raises(ds.Fp8dsError, match="out holds"):
        ds.fp8_bias_grad(g, out=torch.empty(63, dtype=torch.bfloat16), workspace=u8(1 << 16))
    with pytest.raises(ds.Fp8dsError, match="workspace holds"):
        ds.fp8_bias_grad(g, out=torch.empty(64, dtype=torch.bfloat16), workspace=u8(16))


def test_packed_structs_match_the_ctypes_layout():
    """The binding packs fp8_mm_args and fp8_quantize_job with struct; the
    bytes must equal the ctypes structures' (which spell out the header's
    fields), field by field."""
    vals = [0x1000, 0x2000, 0x3000, 1, 0, 2, 3, 17, 33, 65, 2, 80, 96, 112, 4096, 8192, 16384,
            0x4000, 0x5000, 0x6000, 0x7000]
    names = [f[0] for f in ds._MmArgs._fields_]
    c = ds._MmArgs(*vals)
    assert ds._MMARGS.size == ctypes.sizeof(ds._MmArgs)
    assert ds._MMARGS.pack(*vals) == bytes(c)
    for i, name in enumerate(names):           # one field at a time: no two fields swapped
        one = [0] * len(vals)
        one[i] = vals[i]
        assert ds._MMARGS.pack(*one) == bytes(ds._MmArgs(**{name: vals[i]})), name
    jv = [0x8000, 4096, 0x9000, 0xA000, 0xB000]
    assert ds._QJOB.size == ctypes.sizeof(ds._QuantJob)
    assert ds._QJOB.pack(*jv) == bytes(ds._QuantJob(*jv))


def _mm_query_args(layout, m, n, k, batch=1, bias=False, fa=0):
    """fp8_mm arguments of a dense problem at far-apart, aligned addresses
    (the tile query checks the pointers as fp8_mm does but never reads them)."""
    args = ds._MmArgs()
    args.a, args.b, args.c = 1 << 40, 2 << 40, 3 << 40
    args.a_scale_inv, args.b_scale_inv = 4 << 40, 4 << 40
    args.fmt_a, args.fmt_b, args.layout = fa, 0, layout
    args.m, args.n, args.k, args.batch = m, n, k, batch
    a_rows, a_cols = (k, m) if layout == 2 else (m, k)
    b_rows, b_cols = (n, k) if layout == 0 else (k, n)
    args.lda, args.ldb, args.ldc = a_cols, b_cols, n
    args.stride_a, args.stride_b, args.stride_c = a_rows * a_cols, b_rows * b_cols, m * n
    if bias:
        args.bias_kind, args.bias = 1, 5 << 40
    return args


TILE_NONE, TILE_SEPARATE = 64, 65


@pytest.mark.parametrize("shape,bias,tile", [
    ((0, 8192, 8192, 8192, 1), False, 0),     # the bench GEMM: four-wave 256x256
    ((0, 8192, 8192, 8192, 1), True, 6),      # with a bias: the eight-wave 256x256 tile
    ((0, 4096, 3072, 1024, 1), False, 7),     # K <= 1024, partial last round of 256x256 tiles
    ((0, 8192, 3072, 1024, 1), True, 7),      # the same with a bias
    ((0, 4096, 4096, 1024, 1), False, 0),     # one whole round of 256x256 tiles
    ((0, 4096, 4096, 4096, 1), False, 0),
    ((0, 512, 512, 512, 64), False, 7),       # K <= 512: the 128x128 unit tile over whole rounds
    ((1, 2048, 1024, 4096, 1), False, 7),     # 128 tiles of 128x128 with K >= 2048
    ((0, 4096, 1024, 1024, 1), False, 7),     # 256 tiles of 128x128
    ((0, 2048, 1024, 1024, 1), False, 8),     # 128 tiles with K < 2048: the 64x64 unit tile
    ((0, 1024, 1536, 2048, 1), False, 8),
    ((2, 1024, 1024, 4096, 1), False, 8),
    ((0, 0, 64, 64, 1), False, TILE_NONE),    # empty: nothing launched
])
def test_tile_choice(L, shape, bias, tile):
    """The automatic tile choice at the shapes its rules were measured on."""
    layout, m, n, k, batch = shape
    assert L.fp8_mm_tile(ctypes.byref(_mm_query_args(layout, m, n, k, batch, bias))) == tile


@pytest.mark.parametrize("t,n_in,n_out,tile", [
    (4096, 1024, 1024, 7),             # the 12-layer step's O projection at 4096 tokens
    (4096, 4096, 1024, 7),             # its MLP down projection: 320 tiles of 256x256, K = 1024, partial round
    (4096, 1024, 4096, 7),             # its MLP up projection
    (2048, 1024, 1024, 8),             # the O projection at 2048 tokens
    (8192, 1024, 4096, TILE_SEPARATE),  # the rule's eight-wave 256x256 answer: two launches
    (11264, 1024, 11264, TILE_SEPARATE),
])
def test_pair_tile_choice(L, t, n_in, n_out, tile):
    """The pair's tile (dX = G W as NN, dW = G^T X as TN, E5M2 x E4M3), or
    two separate launches."""
    dx = _mm_query_args(1, t, n_in, n_out, fa=1)
    dw = _mm_query_args(2, n_out, n_in, t, fa=1)
    assert L.fp8_mm_pair_tile(ctypes.byref(dx), ctypes.byref(dw)) == tile


def test_tile_query_checks_arguments(L):
    args = _mm_query_args(0, 256, 256, 256)
    args.layout = 7
    assert L.fp8_mm_tile(ctypes.byref(args)) == -1
    nt0 = _mm_query_args(0, 256, 256, 256)
    nt1 = _mm_query_args(0, 128, 256, 256)
    assert L.fp8_mm_pair_tile(ctypes.byref(nt0), ctypes.byref(nt1)) == TILE_SEPARATE   # not NN + TN
    empty = _mm_query_args(1, 0, 256, 256)
    assert L.fp8_mm_pair_tile(ctypes.byref(empty), ctypes.byref(empty)) == TILE_NONE
