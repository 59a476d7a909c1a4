"""MoE dispatch -> grouped GEMM oracle.

[P1] "Los cinco núcleos fusionados", row "Envío MoE + GEMM" ([P3] table
"الحبات الخمس المنصهرة", row for MoE dispatch + GEMM): tokens are routed to
the ranks of their experts (an all-to-all), and the per-expert grouped GEMM
runs on them in the same kernel as they land, with no staging round trip.

Readings (the pages fix none of these):
* Routing picks, per token, the k experts with the largest float32 logits, in
  descending order; equal logits (+0 and -0 are equal) go to the LOWER expert
  id.  Logits must be finite.
* Dispatch is a stable counting sort of the (token, slot) pairs by expert:
  counts[e] = #tokens choosing e, offsets = exclusive prefix sum of counts,
  perm[p] = t*k + j for the p-th pair in (expert ascending, token ascending)
  order.  No gating weight, capacity limit, token dropping or combine step.
* The local experts are ids [expert_begin, expert_begin + L); their rows, in
  dispatch order, form the landing buffer Xs, and Y = Xs_e @ W_e per expert,
  float64 from exact bf16 inputs, rounded once to the output dtype.
"""
import numpy as np

from .numerics import bf16_to_f64, cast_out


def route_topk(logits, k: int) -> np.ndarray:
    """int32[T, k]: indices of the k largest logits per row, ties to the lower index."""
    logits = np.asarray(logits, np.float32)
    if not np.all(np.isfinite(logits)):
        raise ValueError("logits must be finite")
    # A stable sort on the negated value keeps equal values in index order.
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def dispatch(topk: np.ndarray, E: int):
    """(counts int32[E], offsets int32[E+1], perm int32[T*k]) of the stable counting sort."""
    flat = np.asarray(topk, np.int64).ravel()          # pair index t*k + j
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(flat, kind="stable")              # expert asc, then pair index asc
    return counts, offsets.astype(np.int32), perm.astype(np.int32)


def landing_tokens(perm, offsets, k: int, expert_begin: int, L: int) -> np.ndarray:
    """Token id of every landing-buffer row (local experts, dispatch order)."""
    lo, hi = int(offsets[expert_begin]), int(offsets[expert_begin + L])
    return (np.asarray(perm[lo:hi], np.int64) // k)


def grouped_gemm(X, W, offsets, perm, k: int, expert_begin: int, out_dtype="bf16", rows=None):
    """Return (Y64, Y_out) for all landing rows, or only for the landing rows `rows`."""
    L = len(W)
    toks = landing_tokens(perm, offsets, k, expert_begin, L)
    base = int(offsets[expert_begin])
    n = toks.shape[0]
    F = W[0].shape[1]
    sel = np.arange(n) if rows is None else np.asarray(rows, np.int64)
    Y = np.empty((sel.shape[0], F), np.float64)
    for e in range(L):
        lo = int(offsets[expert_begin + e]) - base
        hi = int(offsets[expert_begin + e + 1]) - base
        m = (sel >= lo) & (sel < hi)
        if np.any(m):
            Y[m] = bf16_to_f64(X[toks[sel[m]]]) @ bf16_to_f64(W[e])
    return Y, cast_out(Y, out_dtype)


def moe_dispatch_gemm(X, logits, W, k: int, expert_begin: int, out_dtype="bf16"):
    """Full oracle: routing, dispatch, grouped GEMM."""
    topk = route_topk(logits, k)
    counts, offsets, perm = dispatch(topk, logits.shape[1])
    Y64, Y = grouped_gemm(X, W, offsets, perm, k, expert_begin, out_dtype)
    return dict(topk=topk, counts=counts, offsets=offsets, perm=perm,
                n_local=int(offsets[expert_begin + len(W)] - offsets[expert_begin]),
                Y64=Y64, Y=Y)
