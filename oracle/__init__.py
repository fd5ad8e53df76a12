"""Plain CPU oracle of the delayed-scaling FP8 quantize and the scaled FP8 GEMM.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
and the cpu_baseline leg of bench.py may import, call or execute anything in
this package.  The product path (the HIP library and its Python binding) never
does, and shares no code, table or constant generator with it.

Everything is numpy on the host: float64 for the GEMM, IEEE binary32 for the
amax / history / scale arithmetic, table search for the 8-bit encodings.  Each
function names the passage of the pages it follows and the readings it takes
where the pages are silent.  Every function is pinned by the `-m "not gpu"`
tests in tests/test_oracle_*.py against the format definitions, closed forms,
library casts and brute force; none is "parity unpinned".
"""
from .formats import (E4M3, E5M2, FMAX, IN_BF16, IN_F16, IN_F32, bf16_to_f32, bf16_ulp,
                      decode_fp8, encode_fp8, f64_to_bf16, input_to_f32)
from .scaling import (Ring, advance_ring, amax, next_scale, quantize_step, quantize_values,
                      ring_init)
from .gemm import (NN, NT, TN, bias_values, max_abs_dequant, mm, mm_entries, operand_matrices,
                   tolerance)
from .backward import (DUAL, OUT_BF16, OUT_F32, ROWWISE, TRANSPOSED, bias_grad, bias_grad_tolerance,
                       gradient_values, quantize_step_2d)
from .dynamic import dynamic_ring_after, dynamic_scale, quantize_dynamic

__all__ = [
    "E4M3", "E5M2", "FMAX", "bf16_to_f32", "bf16_ulp", "decode_fp8", "encode_fp8",
    "f64_to_bf16", "Ring", "advance_ring", "amax", "next_scale", "quantize_step", "quantize_values",
    "ring_init", "NT", "NN", "TN", "mm", "mm_entries", "operand_matrices", "tolerance",
    "max_abs_dequant", "bias_values", "IN_BF16", "IN_F16", "IN_F32", "input_to_f32",
    "ROWWISE", "TRANSPOSED", "DUAL", "OUT_BF16", "OUT_F32", "quantize_step_2d", "gradient_values",
    "bias_grad", "bias_grad_tolerance", "dynamic_scale", "quantize_dynamic", "dynamic_ring_after",
]
