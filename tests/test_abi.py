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
