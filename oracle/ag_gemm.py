"""AllGather -> GEMM oracle.

[P1] "Los cinco núcleos fusionados", row "AllGather + GEMM" (and [P3] table
"الحبات الخمس المنصهرة", same row): each rank holds one shard of A; the ranks
gather the other shards while the local GEMM consumes A's tiles as they
arrive; the product is C = A @ B.

Readings:
* The gathered A stacks the shards in RANK order 0..R-1 (AllGather semantics),
  whatever order they arrive in.
* B is row-major [K x N]; C is row-major [M x N] with M = R * m_shard.
* The result is computed in float64 from the exact bf16 values and rounded
  once to the output dtype.
"""
import numpy as np

from .numerics import bf16_to_f64, cast_out
from . import schedule as _schedule


def gather(shards):
    """Gathered A (bf16 bits) in rank order."""
    return np.vstack([np.asarray(s, np.uint16) for s in shards])


def ag_gemm(shards, B, out_dtype="bf16", order=None, delay_ns=None, unit_rows=None):
    """Return (C64, C_out).  The arrival schedule is validated, then ignored."""
    M = sum(s.shape[0] for s in shards)
    if order is not None:
        _schedule.validate(order, delay_ns, M // (unit_rows or shards[0].shape[0]))
    C64 = bf16_to_f64(gather(shards)) @ bf16_to_f64(B)
    return C64, cast_out(C64, out_dtype)


def ag_gemm_rows(shards, B, rows):
    """float64 rows `rows` of C = gather(shards) @ B, computed row by row."""
    m_shard = shards[0].shape[0]
    rows = np.asarray(rows, np.int64)
    A_rows = np.stack([shards[r // m_shard][r % m_shard] for r in rows])
    return bf16_to_f64(A_rows) @ bf16_to_f64(B)


def tile_units(tile_m: int, BM: int, unit_rows: int, M: int):
    """Delivery units a tile of BM rows starting at row tile_m*BM depends on."""
    r0 = tile_m * BM
    r1 = min(M, r0 + BM) - 1
    return r0 // unit_rows, r1 // unit_rows
