"""Comparison rule for floating-point outputs.

Bound: relative Frobenius error <= 1e-3 and max |err| <= 5e-3 * max |ref|.
For bfloat16 outputs the relative Frobenius error is measured against the
correctly rounded reference (rounding alone to bf16 already costs ~1.7e-3
against the unrounded value) and the max error against the unrounded float64
reference; for float32 outputs both are measured against float64.
"""
import numpy as np

from oracle.numerics import f64_to_bf16_bits, bf16_to_f64

REL_FRO = 1e-3
MAX_REL = 5e-3


def errors(y64: np.ndarray, ref64: np.ndarray, out_dtype: str):
    y64 = np.asarray(y64, np.float64)
    ref64 = np.asarray(ref64, np.float64)
    if out_dtype == "bf16":
        ref_fro = bf16_to_f64(f64_to_bf16_bits(ref64))
    else:
        ref_fro = ref64
    den = np.linalg.norm(ref_fro)
    rel_fro = np.linalg.norm(y64 - ref_fro) / (den if den > 0 else 1.0)
    mx = np.max(np.abs(ref64)) if ref64.size else 0.0
    max_err = np.max(np.abs(y64 - ref64)) if ref64.size else 0.0
    return float(rel_fro), float(max_err), float(mx)


def assert_close(y64, ref64, out_dtype, what=""):
    rel_fro, max_err, mx = errors(y64, ref64, out_dtype)
    assert np.all(np.isfinite(y64)), f"{what}: non-finite output"
    assert rel_fro <= REL_FRO, f"{what}: rel-Frobenius {rel_fro:.3e} > {REL_FRO}"
    assert max_err <= MAX_REL * max(mx, 1e-30), f"{what}: max|err| {max_err:.3e} > {MAX_REL}*{mx:.3e}"
    return rel_fro, max_err, mx
