"""MoE combine oracle (the step after the grouped GEMM).

Test infrastructure: only tests/, the package smoke check and bench.py's CPU
baseline use this module; the HIP library never does.

[P1] "Los cinco núcleos fusionados", row "Envío MoE + GEMM": tokens travel
to the ranks of their experts and are multiplied there as they land.  The
pages stop at the expert GEMM; the return of each expert output to its
token's rank and the weighted sum over a token's k experts are not
described.  Readings (none of this is fixed by the pages):
* The gate weight of slot j of token t is the softmax over the token's k
  selected logits, g[t, j] = exp(l[t, e_j]) / sum_i exp(l[t, e_i]).
* out[t] = sum_j g[t, j] * Y_row(t, j), where Y_row(t, j) is the expert
  output of pair (t, j): for a local expert (ids [expert_begin,
  expert_begin + L)) the landing-order row pos - offsets[expert_begin] of
  the local grouped-GEMM output, for any other expert row pos of the peers'
  returned outputs, pos being the pair's dispatch position (perm[pos] =
  t*k + j).
* Inputs bf16 (as the grouped GEMM writes them), exact float64 arithmetic
  here, one final rounding to the output dtype.
"""
import numpy as np

from .numerics import bf16_to_f64, cast_out


def gate_weights(logits, topk) -> np.ndarray:
    """float64[T, k]: softmax over each token's selected logits."""
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(topk, np.int64), axis=1)
    sel = sel - sel.max(axis=1, keepdims=True)
    e = np.exp(sel)
    return e / e.sum(axis=1, keepdims=True)


def pair_positions(perm) -> np.ndarray:
    """int64[T*k]: dispatch position of pair t*k + j (the inverse of perm)."""
    perm = np.asarray(perm, np.int64)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.shape[0])
    return pos


def moe_combine(Y_local, Y_peer, logits, topk, perm, offsets, expert_begin: int, L: int, out_dtype="bf16"):
    """Return (out64 [T, F], out in the output dtype).  Y_local and Y_peer are
    bf16 bit patterns: [>= n_local, F] and [T*k, F]."""
    topk = np.asarray(topk, np.int64)
    T, k = topk.shape
    g = gate_weights(logits, topk)
    pos = pair_positions(perm).reshape(T, k)
    lo, hi = int(offsets[expert_begin]), int(offsets[expert_begin + L])
    yl = bf16_to_f64(Y_local)
    yp = bf16_to_f64(Y_peer)
    F = yp.shape[1]
    out = np.zeros((T, F))
    for j in range(k):
        p = pos[:, j]
        local = (p >= lo) & (p < hi)
        rows = np.empty((T, F))
        rows[local] = yl[p[local] - lo]
        rows[~local] = yp[p[~local]]
        out += g[:, j, None] * rows
    return out, cast_out(out, out_dtype)
