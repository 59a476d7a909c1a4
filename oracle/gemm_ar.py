"""GEMM -> AllReduce oracle.

Test infrastructure: only tests/, the package smoke check and bench.py's CPU
baseline use this module; the HIP library never does.

[P1] "Los cinco núcleos fusionados", row "GEMM + AllReduce" ([P3] table
"الحبات الخمس المنصهرة", same row): compute C = A @ B and reduce the partial
outputs over all ranks in the same launch, each output tile entering the
reduction as soon as it is produced.

Readings:
* As for the reduce-scatter: on one GPU the other R-1 ranks' contributions are
  resident float32 partial sums P_1..P_{R-1}, each [M x N]; this GPU's
  contribution is A @ B.  The reduced result is S = A @ B + P_1 + ... +
  P_{R-1}.
* An all-reduce leaves the whole of S on every rank (a reduce-scatter by row
  block followed by an all-gather of the owner blocks), so the one-GPU share
  delivers S to R outputs, one per rank.  Unlike the reduce-scatter, M need
  not be divisible by R.
* Sums are exact-input float64; each output is rounded once to the output
  dtype.
"""
import numpy as np

from .numerics import bf16_to_f64, cast_out


def gemm_ar(A, B, partials, R: int, out_dtype="f32"):
    """Return (S64, [output of rank r in out dtype] for r < R)."""
    S = bf16_to_f64(A) @ bf16_to_f64(B)
    for P in partials:
        S += np.asarray(P, np.float32).astype(np.float64)
    out = cast_out(S, out_dtype)
    return S, [out.copy() for _ in range(R)]
