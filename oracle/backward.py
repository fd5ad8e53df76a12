"""Neighbours of dX / dW on the backward path: quantize in two orientations and
the bias gradient.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU
baseline leg of the benchmark may import this package.

What the pages fix:
  * the quantize has a transposed and a dual form selected by a layout enum,
    and its tests compare the dual and transposed outputs byte for byte with
    the plain one (AstrAI history of `tests`, entry splitting the quantize
    bindings into quantize / quantize_dual);
  * the bias gradient is the column sum of the output gradient over the rows,
    taken only when the bias needs a gradient; a pre-quantized gradient is
    dequantized before the sum, and gradients are bf16 (fp8.py history
    @f4c44ebf, backward column-sum entry and the bf16-gradient entry).

Readings taken where the pages are silent:
  * the transposed output of an R x C input is the C x R row-major matrix of
    the same codes; the dual form returns both; every form folds the tensor's
    amax into the ring once, exactly as the plain quantize does;
  * a dequantized gradient element is the float32 product dec(code) * s_inv;
  * the bias gradient is the exact column sum rounded once to the output
    type (bf16, or fp32 for callers that keep fp32 gradients).
"""
import numpy as np

from .formats import IN_BF16, decode_fp8, f64_to_bf16, input_to_f32
from .scaling import quantize_step

ROWWISE, TRANSPOSED, DUAL = 0, 1, 2
OUT_BF16, OUT_F32 = 0, 1


def quantize_step_2d(ring, x_bits, rows, cols, layout, kind=IN_BF16):
    """One quantize call on an R x C row-major tensor in the given layout.

    Returns (y or None, y_t or None, new ring): y [rows, cols] the codes in
    the input's order, y_t [cols, rows] the codes of the transpose.  The codes
    and the ring update are those of quantize_step on the same elements.
    """
    x = np.asarray(x_bits).reshape(rows, cols)
    codes, new_ring = quantize_step(ring, x, kind)
    codes = codes.reshape(rows, cols)
    y = codes if layout in (ROWWISE, DUAL) else None
    y_t = np.ascontiguousarray(codes.T) if layout in (TRANSPOSED, DUAL) else None
    return y, y_t, new_ring


def gradient_values(g, kind, fmt=None, scale_inv=None):
    """float32 values of the gradient's elements: raw bf16 / fp16 / fp32 bits
    for kind IN_*, or 8-bit codes (kind None, fmt given) dequantized as the
    float32 product dec(code) * scale_inv."""
    if kind is None:
        dec = decode_fp8(np.asarray(g, dtype=np.uint8), fmt).astype(np.float32)
        with np.errstate(over="ignore", invalid="ignore"):
            return (dec * np.float32(scale_inv)).astype(np.float32)
    return input_to_f32(g, kind)


def bias_grad(g, rows, cols, kind, fmt=None, scale_inv=None):
    """Column sums of the R x C gradient.  Returns (exact sums as float64,
    bf16 bits, float32), the last two each rounded once from the exact sum."""
    v = gradient_values(g, kind, fmt, scale_inv).reshape(rows, cols).astype(np.float64)
    s = v.sum(axis=0) if rows > 0 else np.zeros(cols)
    return s, f64_to_bf16(s), s.astype(np.float32)


def bias_grad_tolerance(g, rows, cols, kind, ref, out_kind, fmt=None, scale_inv=None):
    """Accepted |out - ref| per column for a float32-accumulated sum in any
    order: one unit in the last place of the output type at the reference,
    plus rows * 2^-24 * sum_r |g[r, c]| (the bound of recursive float32
    summation)."""
    v = np.abs(gradient_values(g, kind, fmt, scale_inv).reshape(rows, cols).astype(np.float64))
    acc = rows * 2.0 ** -24 * v.sum(axis=0)
    if out_kind == OUT_BF16:
        from .formats import bf16_ulp
        return bf16_ulp(ref) + acc
    r = np.abs(np.asarray(ref, dtype=np.float32)).astype(np.float64)
    _, ex = np.frexp(np.where(r > 0, r, 1.0))
    ulp = np.ldexp(1.0, np.maximum(ex - 1, -126) - 23)
    return ulp + acc


__all__ = ["ROWWISE", "TRANSPOSED", "DUAL", "OUT_BF16", "OUT_F32", "quantize_step_2d",
           "gradient_values", "bias_grad", "bias_grad_tolerance"]
