"""Python binding of libfp8ds: delayed-scaling FP8 quantize and scaled FP8 GEMM
for MI355X (gfx950).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  The
binding refuses to run when the built library is missing; there is no CPU
fallback.

Entry points (same names as the C ABI in include/fp8ds.h):
    scale_ring_bytes(hist_len)
    scale_ring_init(ring, hist_len, fmt, init_scale=1.0)
    fp8_quantize(x, fmt, ring, out=None)             bf16 / fp16 / fp32 x
    fp8_quantize_batch(xs, fmt, rings, ...)          several tensors, one launch
    fp8_quantize_2d(x, fmt, ring, layout, ...)       row-wise, transposed, dual
    fp8_quantize_dynamic(x, fmt, ring, out=None)     scale from x's own amax
    fp8_bias_grad(g, ..., out=None)                  column sums of a gradient
    fp8_bias_grad_noalloc(g, ..., out=out)           the same without a workspace
    fp8_mm(a, b, ..., out=None)
    fp8_mm_pair(first, second)                       two GEMMs, one launch for dX + dW
plus ScaleRing (a ring in a torch uint8 device tensor), BiasGradWorkspace and
read_ring().
"""
import ctypes
import os
import struct

import torch

E4M3 = 0
E5M2 = 1
NT, NN, TN = 0, 1, 2
BIAS_NONE, BIAS_BF16, BIAS_F32, BIAS_E4M3, BIAS_E5M2 = 0, 1, 2, 3, 4
IN_BF16, IN_F16, IN_F32 = 0, 1, 2
ROWWISE, TRANSPOSED, DUAL = 0, 1, 2
G_BF16, G_F16, G_F32, G_E4M3, G_E5M2 = 0, 1, 2, 3, 4
_IN_TYPE = {torch.bfloat16: IN_BF16, torch.float16: IN_F16, torch.float32: IN_F32}
TILES = {"256x256": 0, "128x128": 1, "64x64": 2, "256x128": 3, "128x256": 4, "256x256w8n": 5, "256x256w8": 6,
         "128x128u": 7, "64x64u": 8}
RING_HIST_OFFSET = 2112   # byte offset of hist[] in a ring (include/fp8ds.h)
RING_GROUPS = 32          # completion-tree scratch lines after the 64-byte header

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8ds.so")
_lib = None


class Fp8dsError(RuntimeError):
    pass


MAX_BATCH = 8             # jobs of one fp8_quantize_batch call


class _QuantJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("numel", ctypes.c_int64), ("ring", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("scale_inv_out", ctypes.c_void_p)]


# The same two structs as packed bytes (the calls pass them by address):
# packing them is several times cheaper per call than filling the ctypes
# structures, which document the layout and serve the ABI tests.
_QJOB = struct.Struct("<QqQQQ")          # fp8_quantize_job, 40 bytes
_MMARGS = struct.Struct("<3Q4i10q4Q")    # fp8_mm_args, 152 bytes


class _MmArgs(ctypes.Structure):
    _fields_ = [
        ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("c", ctypes.c_void_p),
        ("fmt_a", ctypes.c_int), ("fmt_b", ctypes.c_int), ("layout", ctypes.c_int), ("bias_kind", ctypes.c_int),
        ("m", ctypes.c_int64), ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("batch", ctypes.c_int64),
        ("lda", ctypes.c_int64), ("ldb", ctypes.c_int64), ("ldc", ctypes.c_int64),
        ("stride_a", ctypes.c_int64), ("stride_b", ctypes.c_int64), ("stride_c", ctypes.c_int64),
        ("a_scale_inv", ctypes.c_void_p), ("b_scale_inv", ctypes.c_void_p), ("bias", ctypes.c_void_p),
        ("bias_scale_inv", ctypes.c_void_p),
    ]


def lib():
    """The loaded libfp8ds.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise Fp8dsError(f"{LIB_PATH} is missing: build it with "
                             "`python delayed_scaling_amd/build.py` (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        L.fp8_scale_ring_bytes.restype = ctypes.c_size_t
        L.fp8_scale_ring_bytes.argtypes = [ctypes.c_int]
        L.fp8_ring_scale_inv.restype = ctypes.c_void_p
        L.fp8_ring_scale_inv.argtypes = [ctypes.c_void_p]
        L.scale_ring_init.restype = ctypes.c_int
        L.scale_ring_init.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p]
        L.fp8_quantize.restype = ctypes.c_int
        L.fp8_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
        L.fp8_quantize_with_grid.restype = ctypes.c_int
        L.fp8_quantize_with_grid.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        # Struct arguments travel as addresses: packed bytes or byref(ctypes struct).
        L.fp8_mm.restype = ctypes.c_int
        L.fp8_mm.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.fp8_mm_with_tile.restype = ctypes.c_int
        L.fp8_mm_with_tile.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
        L.fp8_mm_with_grid.restype = ctypes.c_int
        L.fp8_mm_with_grid.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.fp8_mm_pair.restype = ctypes.c_int
        L.fp8_mm_pair.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.fp8_mm_tile.restype = ctypes.c_int
        L.fp8_mm_tile.argtypes = [ctypes.c_void_p]
        L.fp8_mm_pair_tile.restype = ctypes.c_int
        L.fp8_mm_pair_tile.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.fp8_quantize_ex.restype = i32
        L.fp8_quantize_ex.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.fp8_quantize_batch.restype = i32
        L.fp8_quantize_batch.argtypes = [vp, i32, i32, i32, vp]
        L.fp8_quantize_2d.restype = i32
        L.fp8_quantize_2d.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
        L.fp8_quantize_dynamic.restype = i32
        L.fp8_quantize_dynamic.argtypes = [vp, i64, i32, i32, vp, vp, vp]
        L.fp8_bias_grad_workspace_bytes.restype = ctypes.c_size_t
        L.fp8_bias_grad_workspace_bytes.argtypes = [i64, i64]
        L.fp8_bias_grad.restype = i32
        L.fp8_bias_grad.argtypes = [vp, i64, i64, i32, vp, i32, vp, vp, vp]
        L.fp8_bias_grad_noalloc.restype = i32
        L.fp8_bias_grad_noalloc.argtypes = [vp, i64, i64, i32, vp, i32, vp, vp]
        L.fp8_last_error.restype = ctypes.c_char_p
        L.fp8_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != 0:
        raise Fp8dsError(f"status {status}: {lib().fp8_last_error().decode()}")


def _stream(stream):
    """The HIP stream to launch on (an address): the given torch stream, else
    the current stream of the current device (read without building a Stream
    object)."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtypes, nbytes, device=True):
    """Check a tensor before its address goes to a kernel: one of `dtypes`,
    contiguous, holding at least the `nbytes` bytes the call touches from its
    first element, and (unless device=False, when the caller checks that for
    all its tensors afterwards with _on_device) in GPU memory.  The C side
    checks sizes against each other but cannot see allocations, so a short
    buffer is caught here, before any launch.  (Attribute reads only: this
    runs on every call.)"""
    if not isinstance(t, torch.Tensor):
        raise Fp8dsError(f"{name} must be a torch tensor" if t is not None else f"{name} is required")
    if t.dtype not in dtypes:
        raise Fp8dsError(f"{name} has dtype {t.dtype}; expected {' or '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise Fp8dsError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise Fp8dsError(f"{name} holds {have} bytes; the call touches {nbytes}")
    if device:
        _on_device((name, t))
    return t


def _on_device(*named):
    """Every given (name, tensor) pair holds GPU memory (None entries skipped)."""
    for name, t in named:
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise Fp8dsError(f"{name} must be a CUDA (HIP) device tensor")


_U8 = (torch.uint8,)
_F32 = (torch.float32,)


def scale_ring_bytes(hist_len):
    return int(lib().fp8_scale_ring_bytes(int(hist_len)))


def scale_ring_init(ring, hist_len, fmt, init_scale=1.0, stream=None):
    """Initialise `ring` (a uint8 device tensor of scale_ring_bytes bytes)."""
    n = scale_ring_bytes(hist_len)
    if n == 0:
        raise Fp8dsError(f"hist_len {hist_len} outside [1, 1024]")
    _need(ring, "ring", _U8, n)
    _check(lib().scale_ring_init(_ptr(ring), int(hist_len), int(fmt), float(init_scale), _stream(stream)))


class ScaleRing:
    """A scale ring held in a torch uint8 device tensor."""

    def __init__(self, hist_len, fmt, init_scale=1.0, device="cuda", stream=None):
        n = scale_ring_bytes(hist_len)
        if n == 0:
            raise Fp8dsError(f"hist_len {hist_len} outside [1, 1024]")
        self.hist_len, self.fmt = int(hist_len), int(fmt)
        self.buf = torch.empty(n, dtype=torch.uint8, device=device)
        scale_ring_init(self.buf, hist_len, fmt, init_scale, stream)
        self._bufp = self.buf.data_ptr()
        self._sinv = lib().fp8_ring_scale_inv(self._bufp)

    def scale_inv_ptr(self):
        """Device address of scale_inv_used (what fp8_mm dequantizes with)."""
        return self._sinv

    def read(self):
        return read_ring(self.buf)


def read_ring(buf):
    """Copy a ring to the host and decode its fields (layout of include/fp8ds.h)."""
    raw = buf.detach().cpu().numpy().tobytes()
    scale, sinv, amax_last, idx, hist_len, fmt, status, _r0, amax_bits, ticket = struct.unpack_from("<fffiiiIIII", raw, 0)
    hist = list(struct.unpack_from(f"<{hist_len}f", raw, RING_HIST_OFFSET)) if 1 <= hist_len <= 1024 else []
    hist_bits = list(struct.unpack_from(f"<{hist_len}I", raw, RING_HIST_OFFSET)) if 1 <= hist_len <= 1024 else []
    groups = struct.unpack_from("<" + "II56x" * RING_GROUPS, raw, 64)
    return {"scale": scale, "scale_inv_used": sinv, "amax_last": amax_last, "idx": idx,
            "hist_len": hist_len, "fmt": fmt, "status": status, "amax_bits": amax_bits,
            "ticket": ticket, "hist": hist, "hist_bits": hist_bits,
            "group_scratch_zero": all(v == 0 for v in groups),
            "scale_bits": struct.unpack_from("<I", raw, 0)[0],
            "scale_inv_used_bits": struct.unpack_from("<I", raw, 4)[0],
            "amax_last_bits": struct.unpack_from("<I", raw, 8)[0]}


def _in_type(x):
    t = _IN_TYPE.get(x.dtype)
    if t is None or not x.is_cuda or not x.is_contiguous():
        raise Fp8dsError("x must be a contiguous bf16, fp16 or fp32 CUDA tensor")
    return t


def _ring_buf(ring):
    """The ring's device buffer; a raw tensor must hold at least a ring of
    history length 1 (its own length is in its device header)."""
    buf = ring.buf if isinstance(ring, ScaleRing) else ring
    return _need(buf, "ring", _U8, scale_ring_bytes(1))


def _codes_out(out, numel, device, name="out"):
    """A uint8 output of numel codes: the given tensor, checked, or a new one."""
    if out is None:
        return torch.empty(numel, dtype=torch.uint8, device=device)
    return _need(out, name, _U8, numel)


def fp8_quantize(x, fmt, ring, out=None, stream=None, max_blocks=None):
    """Quantize x (bf16, fp16 or fp32) with the ring's scale into uint8 codes;
    advances the ring."""
    in_type = _in_type(x)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else \
        _codes_out(out, x.numel(), x.device)
    rbuf = _ring_buf(ring)
    if max_blocks is not None:
        if in_type != IN_BF16:
            raise Fp8dsError("max_blocks is available for bf16 inputs")
        _check(lib().fp8_quantize_with_grid(_ptr(x), x.numel(), int(fmt), _ptr(rbuf), _ptr(out),
                                            int(max_blocks), _stream(stream)))
    elif in_type == IN_BF16:
        _check(lib().fp8_quantize(_ptr(x), x.numel(), int(fmt), _ptr(rbuf), _ptr(out), _stream(stream)))
    else:
        _check(lib().fp8_quantize_ex(_ptr(x), x.numel(), in_type, int(fmt), _ptr(rbuf), _ptr(out),
                                     _stream(stream)))
    return out


def fp8_quantize_batch(xs, fmt, rings, outs=None, scale_inv_outs=None, stream=None):
    """Quantize several tensors of one input type, each with its own ring, in
    one launch (each exactly as fp8_quantize).  scale_inv_outs: optional fp32
    device tensors (or None entries) that receive each job's applied 1/scale.
    Returns the list of code tensors."""
    n = len(xs)
    if n < 1 or n > MAX_BATCH or len(rings) != n:
        raise Fp8dsError(f"fp8_quantize_batch takes 1..{MAX_BATCH} tensors and as many rings")
    in_type = _in_type(xs[0])
    if any(_in_type(x) != in_type for x in xs):
        raise Fp8dsError("fp8_quantize_batch: all tensors must share one dtype")
    if outs is None:
        outs = [torch.empty(x.shape, dtype=torch.uint8, device=x.device) for x in xs]
    if len(outs) != n:
        raise Fp8dsError("fp8_quantize_batch needs one output per tensor")
    for i in range(n):
        _codes_out(outs[i], xs[i].numel(), xs[i].device, f"outs[{i}]")
    sio = scale_inv_outs if scale_inv_outs is not None else [None] * n
    if len(sio) != n:
        raise Fp8dsError("fp8_quantize_batch needs one scale_inv_outs entry (or None) per tensor")
    for i in range(n):
        if sio[i] is not None:
            _need(sio[i], f"scale_inv_outs[{i}]", _F32, 4)
    jobs = b"".join(_QJOB.pack(xs[i].data_ptr(), xs[i].numel(), _ring_buf(rings[i]).data_ptr(), outs[i].data_ptr(),
                               0 if sio[i] is None else sio[i].data_ptr()) for i in range(n))
    _check(lib().fp8_quantize_batch(jobs, n, in_type, int(fmt), _stream(stream)))
    return outs


def fp8_quantize_2d(x, fmt, ring, layout, out=None, out_t=None, stream=None):
    """Quantize a 2-D tensor x [R, C] row-wise, transposed (codes of x.T, [C, R])
    or both (DUAL).  Returns (out, out_t), None for the orientation not made."""
    in_type = _in_type(x)
    if x.dim() != 2:
        raise Fp8dsError("x must be 2-D")
    rows, cols = x.shape
    if layout not in (ROWWISE, TRANSPOSED, DUAL):
        raise Fp8dsError(f"layout {layout} is not ROWWISE, TRANSPOSED or DUAL")
    if layout in (ROWWISE, DUAL):
        out = torch.empty((rows, cols), dtype=torch.uint8, device=x.device) if out is None else \
            _need(out, "out", _U8, rows * cols)
    if layout in (TRANSPOSED, DUAL):
        out_t = torch.empty((cols, rows), dtype=torch.uint8, device=x.device) if out_t is None else \
            _need(out_t, "out_t", _U8, rows * cols)
    _check(lib().fp8_quantize_2d(_ptr(x), rows, cols, in_type, int(fmt), int(layout), _ptr(_ring_buf(ring)),
                                 _ptr(out) if layout != TRANSPOSED else None,
                                 _ptr(out_t) if layout != ROWWISE else None, _stream(stream)))
    return (out if layout != TRANSPOSED else None), (out_t if layout != ROWWISE else None)


def fp8_quantize_dynamic(x, fmt, ring, out=None, stream=None):
    """Dynamic scaling: quantize x with FMAX / amax(x); ring must have hist_len 1
    and afterwards holds scale_inv_used for the GEMM."""
    in_type = _in_type(x)
    out = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else \
        _codes_out(out, x.numel(), x.device)
    _check(lib().fp8_quantize_dynamic(_ptr(x), x.numel(), in_type, int(fmt), _ptr(_ring_buf(ring)), _ptr(out),
                                      _stream(stream)))
    return out


def bias_grad_workspace_bytes(rows, cols):
    return int(lib().fp8_bias_grad_workspace_bytes(int(rows), int(cols)))


class BiasGradWorkspace:
    """Zero-filled device workspace for fp8_bias_grad on [rows, cols] gradients."""

    def __init__(self, rows, cols, device="cuda"):
        self.shape = (int(rows), int(cols))
        self.buf = torch.zeros(max(bias_grad_workspace_bytes(rows, cols), 16), dtype=torch.uint8, device=device)


def fp8_bias_grad(g, rows=None, cols=None, fmt=None, g_scale_inv=None, out_f32=False, out=None,
                  workspace=None, stream=None):
    """Column sums of the gradient g [rows, cols]: bf16 / fp16 / fp32 tensors, or
    uint8 codes of format fmt dequantized with g_scale_inv (ScaleRing, fp32
    device tensor or address).  Returns bf16 [cols] (fp32 with out_f32)."""
    if g.dim() == 2 and rows is None:
        rows, cols = g.shape
    if g.dtype == torch.uint8:
        if fmt is None:
            raise Fp8dsError("uint8 gradients need fmt")
        g_type = G_E4M3 if int(fmt) == E4M3 else G_E5M2
    else:
        g_type = {torch.bfloat16: G_BF16, torch.float16: G_F16, torch.float32: G_F32}.get(g.dtype)
        if g_type is None:
            raise Fp8dsError("g must be bf16, fp16, fp32 or uint8 codes")
    esize = {G_E4M3: 1, G_E5M2: 1, G_F32: 4}.get(g_type, 2)
    _need(g, "g", (g.dtype,), int(rows) * int(cols) * esize, device=False)
    out_dtype = torch.float32 if out_f32 else torch.bfloat16
    if out is None:
        out = torch.empty(int(cols), dtype=out_dtype, device=g.device)
    _need(out, "out", (out_dtype,), int(cols) * (4 if out_f32 else 2), device=False)
    if g_type in (G_E4M3, G_E5M2) and isinstance(g_scale_inv, torch.Tensor):
        _need(g_scale_inv, "g_scale_inv", _F32, 4, device=False)
    if workspace is None:
        workspace = BiasGradWorkspace(rows, cols, g.device)
    wbuf = workspace.buf if isinstance(workspace, BiasGradWorkspace) else workspace
    _need(wbuf, "workspace", _U8, bias_grad_workspace_bytes(rows, cols), device=False)
    _on_device(("g", g), ("out", out), ("g_scale_inv", g_scale_inv), ("workspace", wbuf))
    _check(lib().fp8_bias_grad(_ptr(g), int(rows), int(cols), g_type, _addr(g_scale_inv), int(bool(out_f32)),
                               _ptr(out), _ptr(wbuf), _stream(stream)))
    return out


NOALLOC_MAX_BYTES = 1 << 20   # FP8DS_BIAS_GRAD_NOALLOC_MAX_BYTES


def fp8_bias_grad_noalloc(g, rows=None, cols=None, fmt=None, g_scale_inv=None, out_f32=False,
                          out=None, stream=None):
    """fp8_bias_grad without a workspace (the library's own device scratch),
    for callers that cannot allocate; `out` must then be given.  Shapes whose
    workspace would exceed NOALLOC_MAX_BYTES are refused by the library."""
    if g.dim() == 2 and rows is None:
        rows, cols = g.shape
    if g.dtype == torch.uint8:
        if fmt is None:
            raise Fp8dsError("uint8 gradients need fmt")
        g_type = G_E4M3 if int(fmt) == E4M3 else G_E5M2
    else:
        g_type = {torch.bfloat16: G_BF16, torch.float16: G_F16, torch.float32: G_F32}.get(g.dtype)
        if g_type is None:
            raise Fp8dsError("g must be bf16, fp16, fp32 or uint8 codes")
    esize = {G_E4M3: 1, G_E5M2: 1, G_F32: 4}.get(g_type, 2)
    _need(g, "g", (g.dtype,), int(rows) * int(cols) * esize, device=False)
    out_dtype = torch.float32 if out_f32 else torch.bfloat16
    _need(out, "out", (out_dtype,), int(cols) * (4 if out_f32 else 2), device=False)
    if g_type in (G_E4M3, G_E5M2) and isinstance(g_scale_inv, torch.Tensor):
        _need(g_scale_inv, "g_scale_inv", _F32, 4, device=False)
    _on_device(("g", g), ("out", out), ("g_scale_inv", g_scale_inv))
    _check(lib().fp8_bias_grad_noalloc(_ptr(g), int(rows), int(cols), g_type, _addr(g_scale_inv),
                                       int(bool(out_f32)), _ptr(out), _stream(stream)))
    return out


def _addr(x):
    """Device address of a tensor, a ScaleRing's scale_inv_used or an int
    address; 0 for None."""
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    if isinstance(x, ScaleRing):
        return x._sinv
    return x.data_ptr()


def _extent(rows, cols, ld):
    """Elements one stored [rows][cols] view with leading dimension ld spans."""
    return (rows - 1) * ld + cols if rows > 0 and cols > 0 else 0


def _mm_args(a, b, fmt_a, fmt_b, layout, m, n, k, a_scale_inv, b_scale_inv, bias=None, out=None,
             batch=1, lda=None, ldb=None, ldc=None, stride_a=None, stride_b=None, stride_c=None,
             bias_fmt=None, bias_scale_inv=None):
    """The C argument struct of one GEMM, and its output tensor."""
    a_cols = m if layout == TN else k
    b_cols = k if layout == NT else n
    a_rows = k if layout == TN else m
    b_rows = n if layout == NT else k
    lda = a_cols if lda is None else lda
    ldb = b_cols if ldb is None else ldb
    ldc = n if ldc is None else ldc
    stride_a = a_rows * lda if stride_a is None else stride_a
    stride_b = b_rows * ldb if stride_b is None else stride_b
    stride_c = m * ldc if stride_c is None else stride_c
    dev = a.device if a is not None else b.device
    nb = max(int(batch), 1)
    if out is None:
        out = torch.empty(nb * stride_c if nb > 1 else m * ldc, dtype=torch.bfloat16, device=dev)
    if m > 0 and n > 0:
        # The extents the kernel touches, as the C side computes them
        # (stride 0 broadcasts one entry).
        if k > 0:
            _need(a, "a", _U8, (nb - 1) * stride_a + _extent(a_rows, a_cols, lda), device=False)
            _need(b, "b", _U8, (nb - 1) * stride_b + _extent(b_rows, b_cols, ldb), device=False)
        _need(out, "out", (torch.bfloat16,), 2 * ((nb - 1) * stride_c + _extent(m, n, ldc)), device=False)
    bias_kind = BIAS_NONE
    if bias is not None:
        if bias.dtype == torch.uint8:
            if bias_fmt is None or bias_scale_inv is None:
                raise Fp8dsError("an 8-bit bias needs bias_fmt and bias_scale_inv")
            bias_kind = BIAS_E4M3 if int(bias_fmt) == E4M3 else BIAS_E5M2
        else:
            bias_kind = {torch.bfloat16: BIAS_BF16, torch.float32: BIAS_F32}.get(bias.dtype)
        if bias_kind is None:
            raise Fp8dsError("bias must be bf16, fp32 or uint8 codes")
        _need(bias, "bias", (bias.dtype,), n * bias.element_size(), device=False)
    for nm, sc in (("a_scale_inv", a_scale_inv), ("b_scale_inv", b_scale_inv), ("bias_scale_inv", bias_scale_inv)):
        if isinstance(sc, torch.Tensor):
            _need(sc, nm, _F32, 4, device=False)
    _on_device(("a", a), ("b", b), ("out", out), ("bias", bias), ("a_scale_inv", a_scale_inv),
               ("b_scale_inv", b_scale_inv), ("bias_scale_inv", bias_scale_inv))
    args = _MMARGS.pack(_addr(a), _addr(b), out.data_ptr(), int(fmt_a), int(fmt_b), int(layout), bias_kind,
                        int(m), int(n), int(k), int(batch), int(lda), int(ldb), int(ldc),
                        int(stride_a), int(stride_b), int(stride_c),
                        _addr(a_scale_inv), _addr(b_scale_inv), _addr(bias), _addr(bias_scale_inv))
    return args, out


def fp8_mm(a, b, fmt_a, fmt_b, layout, m, n, k, a_scale_inv, b_scale_inv, bias=None, out=None,
           batch=1, lda=None, ldb=None, ldc=None, stride_a=None, stride_b=None, stride_c=None,
           tile=None, max_workgroups=None, bias_fmt=None, bias_scale_inv=None, stream=None):
    """C = bf16(A @ B * a_scale_inv * b_scale_inv + bias) on uint8 fp8 code tensors.

    a, b: uint8 device tensors holding the stored operands (see include/fp8ds.h
    for the NT/NN/TN storage); a_scale_inv / b_scale_inv: ScaleRing, fp32
    device tensor or device address; bias: bf16 or fp32 device tensor [n] or None.
    Leading dimensions and batch strides default to the dense layout.
    tile forces a tile of the family (TILES name or index); max_workgroups
    bounds the grid so each workgroup runs several output tiles.
    """
    args, out = _mm_args(a, b, fmt_a, fmt_b, layout, m, n, k, a_scale_inv, b_scale_inv, bias, out, batch, lda,
                         ldb, ldc, stride_a, stride_b, stride_c, bias_fmt, bias_scale_inv)
    if tile is None and max_workgroups is None:
        _check(lib().fp8_mm(args, _stream(stream)))
    else:
        t = -1 if tile is None else (TILES[tile] if isinstance(tile, str) else int(tile))
        _check(lib().fp8_mm_with_grid(args, t, int(max_workgroups or 0), _stream(stream)))
    return out


def fp8_mm_pair(first, second, stream=None):
    """Two independent GEMMs issued together (one launch for an NN + TN pair in
    the same formats, as a layer's dX and dW).  first / second: dicts of
    fp8_mm's arguments (a, b, fmt_a, fmt_b, layout, m, n, k, a_scale_inv,
    b_scale_inv and optionally bias, out, ...).  Returns the two outputs."""
    a0, out0 = _mm_args(**first)
    a1, out1 = _mm_args(**second)
    _check(lib().fp8_mm_pair(a0, a1, _stream(stream)))
    return out0, out1


__all__ = ["E4M3", "E5M2", "NT", "NN", "TN", "TILES", "Fp8dsError", "ScaleRing", "fp8_mm", "fp8_mm_pair",
           "fp8_quantize", "fp8_quantize_batch", "fp8_quantize_2d", "fp8_quantize_dynamic", "fp8_bias_grad",
           "fp8_bias_grad_noalloc", "BiasGradWorkspace",
           "bias_grad_workspace_bytes", "lib", "read_ring", "scale_ring_bytes", "scale_ring_init", "LIB_PATH",
           "IN_BF16", "IN_F16", "IN_F32", "ROWWISE", "TRANSPOSED", "DUAL"]
