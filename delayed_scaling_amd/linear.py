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
into a small tensor the backward keeps.  Every arithmetic step runs in the
library's kernels; this module only allocates outputs and orders the calls
on the current stream.
"""
import torch

from . import (E4M3, E5M2, NN, NT, TN, BiasGradWorkspace, ScaleRing, bias_grad_workspace_bytes, fp8_bias_grad,
               fp8_mm, fp8_mm_pair, fp8_quantize, fp8_quantize_batch)


class Fp8LinearState:
    """The three scale rings of one linear layer (x, w: E4M3; g: E5M2) and a
    bias-gradient workspace, created on first use."""

    def __init__(self, hist_len=16, device="cuda"):
        self.ring_x = ScaleRing(hist_len, E4M3, device=device)
        self.ring_w = ScaleRing(hist_len, E4M3, device=device)
        self.ring_g = ScaleRing(hist_len, E5M2, device=device)
        self.workspace = None

    def bias_workspace(self, rows, cols, device):
        if self.workspace is None or self.workspace.buf.numel() < bias_grad_workspace_bytes(rows, cols):
            self.workspace = BiasGradWorkspace(rows, cols, device)
        return self.workspace


class _Fp8LinearFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, w, b, state):
        n_in = x.shape[-1]
        n_out = w.shape[0]
        x2 = x.reshape(-1, n_in).contiguous()
        w2 = w.contiguous()
        t = x2.shape[0]
        s = torch.empty(2, dtype=torch.float32, device=x.device)   # applied 1/scale of X and W
        sx, sw = s[0:1], s[1:2]
        if x2.dtype == w2.dtype:
            x8, w8 = fp8_quantize_batch([x2, w2], E4M3, [state.ring_x, state.ring_w], scale_inv_outs=[sx, sw])
        else:
            x8, = fp8_quantize_batch([x2], E4M3, [state.ring_x], scale_inv_outs=[sx])
            w8, = fp8_quantize_batch([w2], E4M3, [state.ring_w], scale_inv_outs=[sw])
        y = fp8_mm(x8, w8, E4M3, E4M3, NT, t, n_out, n_in, sx, sw, bias=b)
        ctx.save_for_backward(x8, w8, sx, sw)
        ctx.state = state
        ctx.dims = (t, n_in, n_out)
        ctx.x_shape = x.shape
        ctx.has_bias = b is not None
        return y.view(*x.shape[:-1], n_out)

    @staticmethod
    def backward(ctx, gy):
        x8, w8, sx, sw = ctx.saved_tensors
        t, n_in, n_out = ctx.dims
        state = ctx.state
        g2 = gy.reshape(-1, n_out).to(torch.bfloat16).contiguous()
        g8 = fp8_quantize(g2, E5M2, state.ring_g)
        dx = dw = db = None
        dx_args = dict(a=g8, b=w8, fmt_a=E5M2, fmt_b=E4M3, layout=NN, m=t, n=n_in, k=n_out,
                       a_scale_inv=state.ring_g, b_scale_inv=sw)
        dw_args = dict(a=g8, b=x8, fmt_a=E5M2, fmt_b=E4M3, layout=TN, m=n_out, n=n_in, k=t,
                       a_scale_inv=state.ring_g, b_scale_inv=sx)
        if ctx.needs_input_grad[0] and ctx.needs_input_grad[1]:
            dx, dw = fp8_mm_pair(dx_args, dw_args)           # one launch for both
            dx, dw = dx.view(ctx.x_shape), dw.view(n_out, n_in)
        elif ctx.needs_input_grad[0]:
            dx = fp8_mm(**dx_args).view(ctx.x_shape)
        elif ctx.needs_input_grad[1]:
            dw = fp8_mm(**dw_args).view(n_out, n_in)
        if ctx.has_bias and ctx.needs_input_grad[2]:
            db = fp8_bias_grad(g2, t, n_out, workspace=state.bias_workspace(t, n_out, g2.device))
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
