"""Scaled FP8 x FP8 GEMM with fused bias, defined in float64.

Test infrastructure only: nothing outside tests/, the smoke check and the CPU
baseline leg of the benchmark may import this package.

What the pages fix (AstrAI commit history of csrc/kernels/fp8/gemm.cuh and of
astrai/extension/fp8.py):
  * operands are 8-bit floats, products accumulate in fp32 on the device and
    the output is always bf16 (entry dropping the fp8-output template);
  * each operand is dequantized by its own per-tensor scale (scale snapshot
    entry); the bias is added in fp32 before the one bf16 rounding, and N
    tails stay exact (bias-fusion entry);
  * operands may be batched with per-operand batch strides, a zero stride
    broadcasting one matrix over the batch, and transposed views fold into a
    layout tag (3-D operand entry);
  * the linear layer runs its forward on the congruous layout and dX / dW on
    crosswise operands (crosswise-B / crosswise-A entries).

  * an 8-bit stored bias carries its own scale; it becomes a real number
    only at the output stage, once the product has been rescaled by the
    operands' factors (history of test_fp8_mma.py, bias_scale entry).

Definition used here (the reading of "fp32 accumulate" as an approximation of
the exact sum): for every batch b, row m, column n
    acc = sum_k dec(A)[m,k] * dec(B)[k,n]                (float64)
    y   = acc * sa_inv * sb_inv + fl32(bias[n])         (float64)
    out = bf16_round_nearest_even(y)                    (straight from float64)
where an 8-bit bias contributes the float32 product fl32(dec(code) * bias_scale_inv).
Layouts (row-major storage, leading dimensions in elements, batch strides in
elements):
    NT: A stored [M, K] (A[m,k] = a[m*lda + k]),  B stored [N, K] (b[n*ldb + k])
    NN: A stored [M, K],                          B stored [K, N] (b[k*ldb + n])
    TN: A stored [K, M] (A[m,k] = a[k*lda + m]),  B stored [K, N]
"""
import numpy as np

from .formats import bf16_to_f32, bf16_ulp, decode_fp8, f64_to_bf16

NT, NN, TN = 0, 1, 2


def _gather(buf, rows, cols, ld, base, row_major_rows):
    """Index a flat byte buffer as a rows x cols matrix.

    row_major_rows=True: element (i, j) at base + i*ld + j.
    row_major_rows=False: element (i, j) at base + j*ld + i.
    """
    i = np.arange(rows, dtype=np.int64)[:, None]
    j = np.arange(cols, dtype=np.int64)[None, :]
    idx = base + (i * ld + j if row_major_rows else j * ld + i)
    return buf[idx]


def operand_matrices(a, b, layout, m, n, k, lda, ldb, batch_index, stride_a, stride_b):
    """The logical A [M, K] and B [K, N] byte matrices of one batch entry."""
    a = np.asarray(a, dtype=np.uint8).reshape(-1)
    b = np.asarray(b, dtype=np.uint8).reshape(-1)
    base_a = batch_index * stride_a
    base_b = batch_index * stride_b
    if layout == NT:
        am = _gather(a, m, k, lda, base_a, True)
        bm = _gather(b, n, k, ldb, base_b, True).T
    elif layout == NN:
        am = _gather(a, m, k, lda, base_a, True)
        bm = _gather(b, k, n, ldb, base_b, True)
    elif layout == TN:
        am = _gather(a, m, k, lda, base_a, False)
        bm = _gather(b, k, n, ldb, base_b, True)
    else:
        raise ValueError("layout must be NT, NN or TN")
    return am, bm


def bias_values(bias, n, bias_fmt=None, bias_scale_inv=None):
    """The bias as float64 values of float32 numbers: bf16 bits widened, or
    8-bit codes (bias_fmt given) as fl32(dec(code) * bias_scale_inv)."""
    if bias is None:
        return np.zeros(n)
    if bias_fmt is None:
        return bf16_to_f32(np.asarray(bias, dtype=np.uint16)).astype(np.float64)
    dec = decode_fp8(np.asarray(bias, dtype=np.uint8), bias_fmt).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        return (dec * np.float32(bias_scale_inv)).astype(np.float32).astype(np.float64)


def mm(a, b, fmt_a, fmt_b, layout, m, n, k, lda, ldb, sa_inv, sb_inv,
       bias=None, batch=1, stride_a=0, stride_b=0, bias_fmt=None, bias_scale_inv=None):
    """Full result.  Returns (y float64 [batch, m, n], out bf16 bits [batch, m, n]).

    sa_inv / sb_inv are the float32 dequantization multipliers (the reciprocal
    of the scale each operand was quantized with); bias is bf16 bits [n], or
    8-bit codes [n] with bias_fmt and bias_scale_inv, or None.
    """
    batch = max(int(batch), 1)
    y = np.zeros((batch, m, n), dtype=np.float64)
    bias64 = bias_values(bias, n, bias_fmt, bias_scale_inv)
    for bi in range(batch):
        am, bm = operand_matrices(a, b, layout, m, n, k, lda, ldb, bi, stride_a, stride_b)
        acc = decode_fp8(am, fmt_a) @ decode_fp8(bm, fmt_b) if k > 0 else np.zeros((m, n))
        y[bi] = acc * np.float64(np.float32(sa_inv)) * np.float64(np.float32(sb_inv)) + bias64[None, :]
    return y, f64_to_bf16(y)


def mm_entries(a, b, fmt_a, fmt_b, layout, m, n, k, lda, ldb, sa_inv, sb_inv,
               bi, mi, ni, bias=None, stride_a=0, stride_b=0, bias_fmt=None, bias_scale_inv=None):
    """Selected entries (bi[t], mi[t], ni[t]) of the same definition, one dot
    product each, for outputs too large to form whole."""
    a = np.asarray(a, dtype=np.uint8).reshape(-1)
    b = np.asarray(b, dtype=np.uint8).reshape(-1)
    bi = np.asarray(bi, dtype=np.int64)
    mi = np.asarray(mi, dtype=np.int64)
    ni = np.asarray(ni, dtype=np.int64)
    kk = np.arange(k, dtype=np.int64)[None, :]
    base_a = (bi * stride_a)[:, None]
    base_b = (bi * stride_b)[:, None]
    if layout in (NT, NN):
        ia = base_a + mi[:, None] * lda + kk
    else:
        ia = base_a + kk * lda + mi[:, None]
    if layout == NT:
        ib = base_b + ni[:, None] * ldb + kk
    else:
        ib = base_b + kk * ldb + ni[:, None]
    acc = (decode_fp8(a[ia], fmt_a) * decode_fp8(b[ib], fmt_b)).sum(axis=1)
    bias64 = (np.zeros(len(ni)) if bias is None else
              bias_values(np.asarray(bias)[ni], len(ni), bias_fmt, bias_scale_inv))
    y = acc * np.float64(np.float32(sa_inv)) * np.float64(np.float32(sb_inv)) + bias64
    return y, f64_to_bf16(y)


def tolerance(ref_bits, k, max_abs_a, max_abs_b):
    """Accepted |out - ref| per element: 2 bf16 ulps of the reference plus
    1e-3 * sqrt(K) * max|A_deq| * max|B_deq| (maxima over the whole dequantized
    operands of the call)."""
    return 2.0 * bf16_ulp(ref_bits) + 1e-3 * np.sqrt(max(k, 0)) * max_abs_a * max_abs_b


def max_abs_dequant(codes, fmt, s_inv):
    """max |dec(code) * s_inv| over an operand (NaN-free operands)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if c.size == 0:
        return 0.0
    present = np.flatnonzero(np.bincount(c, minlength=256)).astype(np.uint8)
    vals = np.abs(decode_fp8(present, fmt))
    return float(np.nanmax(vals)) * float(np.float32(s_inv))


__all__ = ["NT", "NN", "TN", "mm", "mm_entries", "tolerance", "operand_matrices",
           "max_abs_dequant", "bias_values"]
