"""Delayed per-tensor scaling: amax, the amax-history ring and the quantize step.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU
baseline leg of the benchmark may import this package.

What the pages fix (AstrAI commit history of astrai/extension/fp8.py,
@4dc5e923 and @f4c44ebf):
  * each operand (x, w, g) owns a separate ring holding an amax history, a
    write index and the scale; one ring per operand keeps the amax of one
    tensor out of another's scale (FP8TensorMeta entries);
  * a single quantize call also updates the ring: the new amax goes into the
    slot the index points at, the history is reduced to one number and the
    scale for the following call is derived from it (ring-finalize entry);
  * the amax is taken over the values before quantization, in fp32 (the amax
    fix entry: taking it after the cast pins it near 448 and the scale at 1);
  * the GEMM dequantizes with the scale the quantize actually applied, kept
    apart from the newly published one (scale snapshot entry).

Readings taken where the pages are silent:
  * direction: q = cast(x * scale) and next scale = FMAX / window_max;
  * the window reduction is the maximum over all hist slots; unwritten slots
    hold 0 and never win;
  * the next scale is published only when window_max is finite and positive
    and FMAX / window_max is finite; otherwise the old scale stays;
  * no margin and no power-of-two rounding of the scale;
  * a call on an empty tensor leaves the ring unchanged;
  * NaN inputs propagate into amax (their |x| bit pattern exceeds +inf's).
"""
from dataclasses import dataclass, field

import numpy as np

from .formats import E4M3, E5M2, FMAX, IN_BF16, encode_fp8, input_to_f32


@dataclass
class Ring:
    """Oracle state of one amax-history ring."""
    fmt: int
    hist_len: int
    scale: np.float32
    scale_inv_used: np.float32
    amax_last: np.float32
    idx: int = 0
    hist: np.ndarray = field(default=None)

    def copy(self):
        return Ring(self.fmt, self.hist_len, np.float32(self.scale),
                    np.float32(self.scale_inv_used), np.float32(self.amax_last),
                    int(self.idx), self.hist.copy())


def ring_init(hist_len, fmt, init_scale=1.0):
    """Fresh ring: empty history, scale = init_scale, 1/init_scale recorded."""
    if fmt not in (E4M3, E5M2):
        raise ValueError("bad fmt")
    if not 1 <= hist_len <= 1024:
        raise ValueError("hist_len must be in [1, 1024]")
    s = np.float32(init_scale)
    if not (np.isfinite(s) and s > 0):
        raise ValueError("init_scale must be finite and positive")
    return Ring(fmt, hist_len, s, np.float32(1.0) / s, np.float32(0.0), 0,
                np.zeros(hist_len, dtype=np.float32))


def amax(x_bits, kind=IN_BF16):
    """max |x| over the tensor, taken on the float32 bit patterns of |x|.

    |x| as float32 is non-negative, so its bit pattern orders like its value,
    with any NaN above +inf.  Exact and independent of order.  x holds raw
    bits of the input type `kind` (bf16 by default).
    """
    x = np.asarray(x_bits).reshape(-1)
    if x.size == 0:
        return np.float32(0.0)
    mag_bits = input_to_f32(x, kind).view(np.uint32) & np.uint32(0x7FFFFFFF)
    return np.uint32(mag_bits.max()).view(np.float32)


def quantize_values(x_bits, scale, fmt, kind=IN_BF16):
    """Codes of cast(fl32(x) * scale): one float32 multiply, then encode.

    A NaN element keeps the sign of the input element.
    """
    x = input_to_f32(np.asarray(x_bits), kind)
    with np.errstate(over="ignore", invalid="ignore"):
        v = x * np.float32(scale)                 # IEEE binary32 product, nearest-even
    v = np.where(np.isnan(x), np.copysign(np.float32(np.nan), x), v).astype(np.float32)
    return encode_fp8(v, fmt)


def next_scale(hist, fmt, old_scale):
    """Scale published from a history window (see the readings above)."""
    w = np.asarray(hist, dtype=np.float32).view(np.uint32).max().view(np.float32)
    if not (np.isfinite(w) and w > 0):
        return np.float32(old_scale)
    with np.errstate(over="ignore", divide="ignore"):
        t = np.float32(FMAX[fmt]) / w                 # IEEE binary32 quotient
    return t if np.isfinite(t) else np.float32(old_scale)


def advance_ring(ring, a):
    """The ring update of one quantize call whose tensor had amax `a`:
    store a in hist[idx] and step idx; derive the next scale from the
    window's maximum; record 1/scale_used and the amax.  Returns the new
    ring."""
    r = ring.copy()
    s_used = np.float32(r.scale)
    r.hist[r.idx] = np.float32(a)
    r.idx = (r.idx + 1) % r.hist_len
    r.scale = next_scale(r.hist, r.fmt, s_used)
    r.scale_inv_used = np.float32(1.0) / s_used
    r.amax_last = np.float32(a)
    return r


def quantize_step(ring, x_bits, kind=IN_BF16):
    """One delayed-scaling quantize call.

    Returns (codes, new ring).  In order: quantize with the current scale,
    then advance the ring with the tensor's amax (advance_ring).
    """
    x = np.asarray(x_bits)
    if x.size == 0:
        return np.zeros(x.shape, dtype=np.uint8), ring.copy()
    codes = quantize_values(x, np.float32(ring.scale), ring.fmt, kind)
    return codes, advance_ring(ring, amax(x, kind))


__all__ = ["Ring", "ring_init", "amax", "quantize_values", "next_scale", "advance_ring",
           "quantize_step", "E4M3", "E5M2", "FMAX"]
