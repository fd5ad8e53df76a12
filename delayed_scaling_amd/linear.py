"""An FP8 linear layer with delayed scaling, as a thin torch.autograd.Function
over the library's C ABI (AstrAI history of astrai/extension/fp8.py @4dc5e923:
the layer's forward and backward live in one autograd Function whose backward
reads only what the forward saved, so it runs in FP8 wherever it is called).

Forward   y  = X W^T (+ b):  X -> E4M3 (ring x), W -> E4M3 (ring w), NT GEMM.
Backward  G -> E5M2 (ring g);  dX = G W (NN on the forward's W codes) and
          dW = G^T X (TN on the forward's X codes) in one launch, db = column
          sums of G (only when the bias needs a gradient).
The forward's dequantization scales are kept aside when the forward runs
(fp8.py @f4c44ebf, forward-carries-scale entry), so a later forward on the
same rings cannot change what the backward dequantizes with: X and W are
quantized in one batched launch that also writes both applied 1/scale values
next to the codes, in the one buffer the backward keeps.  Every arithmetic step runs in the
library's kernels; this module only allocates outputs and orders the calls
on the current stream.

The layer calls the C ABI directly with packed argument structs: every
buffer but x, w, b and the incoming gradient is one it allocated itself with
the size the call needs, so the per-tensor checks of the general binding
(which cost more host time than the launches) reduce to those four tensors.
"""
import torch

from . import (_IN_TYPE, _MMARGS, _QJOB, BIAS_BF16, BIAS_F32, BIAS_NONE, E4M3, E5M2, G_BF16, NN, NT, TN,
               BiasGradWorkspace, Fp8dsError, ScaleRing, _check, _stream, bias_grad_workspace_bytes, lib)


class Fp8LinearState:
    """The three scale rings of one linear layer (x, w: E4M3; g: E5M2) and a
    bias-gradient workspace, created on first use."""

    def __init__(self, hist_len=16, device="cuda"):
        self.ring_x = ScaleRing(hist_len, E4M3, device=device)
        self.ring_w = ScaleRing(hist_len, E4M3, device=device)
        self.ring_g = ScaleRing(hist_len, E5M2, device=device)
        self.workspace = None
        self._ws_shape = None

    def bias_workspace(self, rows, cols, device):
        if self._ws_shape != (rows, cols):
            if self.workspace is None or self.workspace.buf.numel() < bias_grad_workspace_bytes(rows, cols):
                self.workspace = BiasGradWorkspace(rows, cols, device)
            self._ws_shape = (rows, cols)
        return self.workspace


def _input(t, name, dev):
    """A caller's tensor going to a kernel: bf16 / fp16 / fp32, on the GPU of
    the layer, made contiguous."""
    if t.dtype not in _IN_TYPE:
        raise Fp8dsError(f"{name} must be bf16, fp16 or fp32, not {t.dtype}")
    if t.device != dev:
        raise Fp8dsError(f"{name} is on {t.device}; the layer runs on {dev}")
    return t if t.is_contiguous() else t.contiguous()


def _mm(a, b, c, fmt_a, layout, m, n, k, sa, sb, bias=None, bias_kind=BIAS_NONE):
    """The argument struct of one dense GEMM (formats fmt_a x E4M3) over
    contiguous operands the layer allocated (a, b, c: device addresses)."""
    a_cols = m if layout == TN else k
    b_cols = k if layout == NT else n
    a_rows = k if layout == TN else m
    b_rows = n if layout == NT else k
    return _MMARGS.pack(a, b, c, fmt_a, E4M3, layout, bias_kind, m, n, k, 1,
                        a_cols, b_cols, n, a_rows * a_cols, b_rows * b_cols, m * n, sa, sb,
                        0 if bias is None else bias.data_ptr(), 0)


def _codes_layout(t, n_in, n_out):
    """Byte offsets of the forward's saved buffer: X's codes [t, n_in], W's
    codes [n_out, n_in], then the two applied 1/scale values (each piece
    256-byte aligned).  One allocation instead of three: the layer's host
    time per call is mostly fixed costs like these."""
    wo = (t * n_in + 255) & ~255
    so = wo + ((n_out * n_in + 255) & ~255)
    return wo, so, so + 8


class _Fp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, b, state):
        n_in = x.shape[-1]
        n_out = w.shape[0]
        if w.dim() != 2 or w.shape[1] != n_in:
            raise Fp8dsError(f"weight {tuple(w.shape)} does not take inputs of {n_in} features")
        dev = w.device
        x2 = _input(x.reshape(-1, n_in), "x", dev)
        w2 = _input(w, "weight", dev)
        t = x2.shape[0]
        L, st = lib(), _stream(None)
        wo, so, nbytes = _codes_layout(t, n_in, n_out)
        saved = torch.empty(nbytes, dtype=torch.uint8, device=dev)   # X codes | W codes | 1/scale of X, W
        x8 = saved.data_ptr()
        w8, sp = x8 + wo, x8 + so
        jx = _QJOB.pack(x2.data_ptr(), x2.numel(), state.ring_x._bufp, x8, sp)
        jw = _QJOB.pack(w2.data_ptr(), w2.numel(), state.ring_w._bufp, w8, sp + 4)
        if x2.dtype == w2.dtype:
            _check(L.fp8_quantize_batch(jx + jw, 2, _IN_TYPE[x2.dtype], E4M3, st))
        else:
            _check(L.fp8_quantize_batch(jx, 1, _IN_TYPE[x2.dtype], E4M3, st))
            _check(L.fp8_quantize_batch(jw, 1, _IN_TYPE[w2.dtype], E4M3, st))
        bias_kind = BIAS_NONE
        if b is not None:
            bias_kind = {torch.bfloat16: BIAS_BF16, torch.float32: BIAS_F32}.get(b.dtype)
            if bias_kind is None or b.device != dev or b.numel() != n_out:
                raise Fp8dsError("bias must be a bf16 or fp32 tensor of out_features elements on the layer's GPU")
            b = b if b.is_contiguous() else b.contiguous()
        y = torch.empty((t, n_out), dtype=torch.bfloat16, device=dev)
        _check(L.fp8_mm(_mm(x8, w8, y.data_ptr(), E4M3, NT, t, n_out, n_in, sp, sp + 4, b, bias_kind), st))
        ctx.save_for_backward(saved)
        ctx.state = state
        ctx.dims = (t, n_in, n_out)
        ctx.x_shape = x.shape
        ctx.has_bias = b is not None
        return y.view(*x.shape[:-1], n_out)

    @staticmethod
    def backward(ctx, gy):
        saved, = ctx.saved_tensors
        t, n_in, n_out = ctx.dims
        state = ctx.state
        dev = saved.device
        wo, so, _ = _codes_layout(t, n_in, n_out)
        x8 = saved.data_ptr()
        w8, sp = x8 + wo, x8 + so
        g2 = gy.reshape(-1, n_out)
        if g2.dtype != torch.bfloat16 or not g2.is_contiguous():
            g2 = g2.to(torch.bfloat16).contiguous()
        L, st = lib(), _stream(None)
        g8t = torch.empty((t, n_out), dtype=torch.uint8, device=dev)
        g8 = g8t.data_ptr()
        _check(L.fp8_quantize(g2.data_ptr(), g2.numel(), E5M2, state.ring_g._bufp, g8, st))
        sg = state.ring_g._sinv
        dx = dw = db = None
        need_x, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if need_x:
            dx = torch.empty((t, n_in), dtype=torch.bfloat16, device=dev)
            ax = _mm(g8, w8, dx.data_ptr(), E5M2, NN, t, n_in, n_out, sg, sp + 4)
        if need_w:
            dw = torch.empty((n_out, n_in), dtype=torch.bfloat16, device=dev)
            aw = _mm(g8, x8, dw.data_ptr(), E5M2, TN, n_out, n_in, t, sg, sp)
        if need_x and need_w:
            _check(L.fp8_mm_pair(ax, aw, st))                   # one launch for both
        elif need_x:
            _check(L.fp8_mm(ax, st))
        elif need_w:
            _check(L.fp8_mm(aw, st))
        if dx is not None:
            dx = dx.view(ctx.x_shape)
        if ctx.has_bias and ctx.needs_input_grad[2]:
            ws = state.bias_workspace(t, n_out, dev)
            db = torch.empty(n_out, dtype=torch.bfloat16, device=dev)
            _check(L.fp8_bias_grad(g2.data_ptr(), t, n_out, G_BF16, None, 0, db.data_ptr(), ws.buf.data_ptr(), st))
        return dx, dw, db, None


def fp8_linear(x, weight, bias, state):
    """y = x @ weight.T + bias through FP8 with delayed scaling (bf16 in and out)."""
    return _Fp8LinearFn.apply(x, weight, bias, state)


class Fp8Linear(torch.nn.Module):
    """Drop-in linear layer (bf16 parameters) computing in FP8.  in_features
    and out_features must be multiples of 16 (the GEMM's 16-byte row
    alignment); any number of tokens."""

    def __init__(self, in_features, out_features, bias=True, hist_len=16, device="cuda"):
        super().__init__()
        self.weight = torch.nn.Parameter(torch.empty(out_features, in_features, dtype=torch.bfloat16,
                                                     device=device))
        self.bias = (torch.nn.Parameter(torch.zeros(out_features, dtype=torch.bfloat16, device=device))
                     if bias else None)
        torch.nn.init.normal_(self.weight, std=in_features ** -0.5)
        self.state = Fp8LinearState(hist_len, device)

    def forward(self, x):
        return fp8_linear(x, self.weight, self.bias, self.state)


__all__ = ["Fp8Linear", "Fp8LinearState", "fp8_linear"]
