"""The dynamic-scaling recipe: each tensor is scaled by its own amax.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU
baseline leg of the benchmark may import this package.

What the pages fix: besides delayed scaling there is a dynamic recipe that
keeps no history: its scales are measured inline from the tensor being
quantized (fp8.py history @4dc5e923, entry that skips the meta allocation on
the dynamic path; history of `tests`, entry merging the two recipes into one
dataclass with a dynamic flag).

Readings taken where the pages are silent:
  * scale = fl32(FMAX / amax(x)) when amax is finite and positive and the
    quotient is finite, otherwise 1 (an all-zero, infinite or NaN tensor has
    no usable amax);
  * the codes are quantize_values(x, scale) and the GEMM dequantizes with
    fl32(1 / scale), as on the delayed path;
  * as a length-1 scale ring, a call leaves hist = [amax], the published
    scale equal to the scale used, scale_inv_used = fl32(1 / scale) and
    amax_last = amax.
"""
import numpy as np

from .formats import FMAX, IN_BF16
from .scaling import Ring, amax, quantize_values


def dynamic_scale(a, fmt):
    """Scale of a tensor with amax a."""
    a = np.float32(a)
    if not (np.isfinite(a) and a > 0):
        return np.float32(1.0)
    with np.errstate(over="ignore", divide="ignore"):
        t = np.float32(FMAX[fmt]) / a
    return t if np.isfinite(t) else np.float32(1.0)


def quantize_dynamic(x_bits, fmt, kind=IN_BF16):
    """Returns (codes, scale, scale_inv, amax) of one dynamic quantize."""
    x = np.asarray(x_bits)
    a = amax(x, kind)
    s = dynamic_scale(a, fmt)
    codes = quantize_values(x, s, fmt, kind) if x.size else np.zeros(x.shape, np.uint8)
    return codes, s, np.float32(1.0) / s, a


def dynamic_ring_after(x_bits, fmt, kind=IN_BF16):
    """The length-1 ring a dynamic call leaves behind (see the readings)."""
    _, s, s_inv, a = quantize_dynamic(x_bits, fmt, kind)
    return Ring(fmt, 1, s, s_inv, np.float32(a), 0, np.array([a], dtype=np.float32))


__all__ = ["dynamic_scale", "quantize_dynamic", "dynamic_ring_after"]
