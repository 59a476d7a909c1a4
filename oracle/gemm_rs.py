"""GEMM -> ReduceScatter oracle.

[P1] "Los cinco núcleos fusionados", row "GEMM + ReduceScatter" ([P3] table
"الحبات الخمس المنصهرة", same row): compute C = A @ B, then reduce the output
across ranks and scatter it, each output tile being reduced and sent to the
rank that owns it as soon as it is produced.

Readings:
* On one GPU the other R-1 ranks' contributions are resident float32 partial
  sums P_1..P_{R-1}, each [M x N]; this GPU's contribution is A @ B.
* The reduced result is S = A @ B + P_1 + ... + P_{R-1}; ownership is by row
  block: owner r receives rows [r*M/R, (r+1)*M/R) of S.  All R owner blocks are
  produced (the full reduction sliced by owner).
* Sums are exact-input float64; each owner block is rounded once to the
  output dtype (float32 by default, the dtype of the partial sums).
* The partial sums may arrive over time, in units of (peer, row block): the
  reduction of a tile waits for the units under its rows.  As for the
  AllGather's chunks, the arrival schedule decides only WHEN a tile is
  reduced, never the result, so it is validated here and otherwise ignored.
"""
import numpy as np

from .numerics import bf16_to_f64, cast_out
from . import schedule as _schedule


def owner_of_row(row: int, M: int, R: int) -> int:
    return int(row) // (M // R)


def partial_units(M: int, R: int, unit_rows: int) -> int:
    """Number of (peer, row block) delivery units of the R-1 partial sums."""
    if M % unit_rows:
        raise _schedule.ScheduleError("unit_rows must divide M")
    return (R - 1) * (M // unit_rows)


def unit_of(peer: int, row: int, M: int, unit_rows: int) -> int:
    """Unit id of row `row` of partial `peer` (1..R-1): peer-major, then row block."""
    return (peer - 1) * (M // unit_rows) + int(row) // unit_rows


def gemm_rs(A, B, partials, R: int, out_dtype="f32", order=None, delay_ns=None, unit_rows=None):
    """Return (S64, [owner block float64], [owner block in out dtype]).  An
    arrival schedule of the partial sums (order, delay_ns over the units of
    unit_rows rows) is validated, then ignored."""
    M = A.shape[0]
    if M % R:
        raise ValueError("M must be divisible by R")
    if order is not None:
        _schedule.validate(order, delay_ns, partial_units(M, R, unit_rows))
    S = bf16_to_f64(A) @ bf16_to_f64(B)
    for P in partials:
        S += np.asarray(P, np.float32).astype(np.float64)
    mb = M // R
    blocks = [S[r * mb:(r + 1) * mb] for r in range(R)]
    return S, blocks, [cast_out(b, out_dtype) for b in blocks]


def gemm_rs_rows(A, B, partials, rows):
    """float64 rows `rows` of the fully reduced S, computed row by row."""
    rows = np.asarray(rows, np.int64)
    S = bf16_to_f64(A[rows]) @ bf16_to_f64(B)
    for P in partials:
        S += np.asarray(P[rows], np.float32).astype(np.float64)
    return S


def tile_owner(tile_m: int, BM: int, M: int, R: int) -> int:
    """Owner of an output tile whose first row is tile_m*BM (tiles never straddle owners)."""
    return owner_of_row(tile_m * BM, M, R)
