"""Pins of the MoE routing / dispatch / grouped-GEMM oracle: brute-force
top-k with explicit tie-breaking, a textbook stable counting sort, dispatch
invariants and fsum / exact-integer grouped GEMM."""
import math

import numpy as np
import pytest

import oracle.moe as om
from oracle.numerics import bf16_to_f64
import workloads as wl


def brute_topk(logits, k):
    """Pure Python: repeatedly take the largest remaining value, lowest index on ties."""
    out = []
    for row in logits.tolist():
        left = list(range(len(row)))
        pick = []
        for _ in range(k):
            best = left[0]
            for e in left[1:]:
                if row[e] > row[best]:          # strict: equal keeps the lower index
                    best = e
            pick.append(best)
            left.remove(best)
        out.append(pick)
    return np.array(out, np.int32)


def pin_topk(fn, seed=21):
    rng = np.random.default_rng(seed)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.0], np.float32)
    L = vals[rng.integers(0, len(vals), size=(64, 12))]
    return np.array_equal(fn(L, 5), brute_topk(L, 5))


def pin_constant(fn):
    L = np.full((10, 32), 0.25, np.float32)
    L[::2] = -0.0
    L[1::4] = 0.0
    return np.array_equal(fn(L, 8), np.tile(np.arange(8, dtype=np.int32), (10, 1)))


def test_topk_brute_force_with_ties_and_signed_zero():
    assert pin_topk(om.route_topk)


def test_constant_logits_pick_lowest_ids():
    assert pin_constant(om.route_topk)


def test_topk_on_zipf_logits_dominates_unchosen():
    w = wl.make_moe(300, 8, 64, 8, 4, 8, seed=22)
    t = om.route_topk(w.logits, 8)
    for i in range(300):
        chosen = w.logits[i, t[i]]
        rest = np.delete(w.logits[i], t[i])
        assert np.all(np.diff(chosen) <= 0)            # descending
        assert chosen.min() >= rest.max()
        assert len(set(t[i].tolist())) == 8


def test_nonfinite_logits_rejected():
    L = np.zeros((2, 4), np.float32)
    L[1, 2] = np.nan
    with pytest.raises(ValueError):
        om.route_topk(L, 2)


def test_dispatch_k1_is_textbook_counting_sort():
    rng = np.random.default_rng(23)
    T, E = 200, 7
    topk = rng.integers(0, E, size=(T, 1)).astype(np.int32)
    counts, offsets, perm = om.dispatch(topk, E)
    ref = sorted(range(T), key=lambda t: (int(topk[t, 0]), t))
    assert perm.tolist() == ref
    assert counts.tolist() == [int((topk == e).sum()) for e in range(E)]
    assert offsets.tolist() == [0] + np.cumsum(counts).tolist()


def check_dispatch_invariants(topk, counts, offsets, perm, E):
    T, k = topk.shape
    assert counts.sum() == T * k
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.sort(perm), np.arange(T * k))          # bijection
    for e in range(E):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert np.all(topk.ravel()[seg] == e)
        toks = seg // k
        assert np.all(np.diff(toks) > 0)                             # ascending, distinct


def test_dispatch_invariants_on_zipf_routing():
    w = wl.make_moe(512, 8, 256, 8, 32, 8, seed=24)
    topk = om.route_topk(w.logits, 8)
    counts, offsets, perm = om.dispatch(topk, 256)
    check_dispatch_invariants(topk, counts, offsets, perm, 256)
    # Zipf popularity: expert 0 is chosen far more often than expert 255
    assert counts[0] > 4 * max(counts[255], 1)


def test_grouped_gemm_fsum_brute_force():
    w = wl.make_moe(24, 16, 8, 3, 4, 5, seed=25, expert_begin=2)
    r = om.moe_dispatch_gemm(w.X, w.logits, w.W, 3, 2, "f32")
    toks = om.landing_tokens(r["perm"], r["offsets"], 3, 2, 4)
    base = r["offsets"][2]
    for q, t in enumerate(toks):
        pair = r["perm"][base + q]
        e = r["topk"].ravel()[pair] - 2
        for j in range(5):
            ref = math.fsum(bf16_to_f64(w.X[t]) * bf16_to_f64(w.W[e][:, j]))
            assert abs(r["Y64"][q, j] - ref) <= 1e-14 * (1 + abs(ref))


def test_grouped_gemm_integer_exact_and_rows_helper():
    w = wl.make_moe(40, 24, 16, 4, 6, 7, seed=26, dist="int")
    r = om.moe_dispatch_gemm(w.X, w.logits, w.W, 4, 0, "f32")
    toks = om.landing_tokens(r["perm"], r["offsets"], 4, 0, 6)
    Xi = bf16_to_f64(w.X).astype(np.int64)
    for e in range(6):
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        ref = Xi[toks[lo:hi]] @ bf16_to_f64(w.W[e]).astype(np.int64)
        assert np.array_equal(r["Y64"][lo:hi], ref.astype(np.float64))
    rows = [0, r["n_local"] - 1, 3]
    Ys, _ = om.grouped_gemm(w.X, w.W, r["offsets"], r["perm"], 4, 0, "f32", rows=rows)
    assert np.array_equal(Ys, r["Y64"][rows])


# ---- mutants ----
def _mut_tie_high(logits, k):
    L = np.asarray(logits, np.float64)[:, ::-1]
    o = np.argsort(-L, axis=1, kind="stable")[:, :k]
    return (L.shape[1] - 1 - o).astype(np.int32)


def _mut_unstable_zero(logits, k):
    # sorts on raw bits: -0 would rank below +0
    b = np.asarray(logits, np.float32).view(np.int32).astype(np.int64)
    key = np.where(b < 0, -(b & 0x7FFFFFFF) - 1, b)
    return np.argsort(-key, axis=1, kind="stable")[:, :k].astype(np.int32)


def test_mutants_are_caught():
    assert not (pin_topk(_mut_tie_high) and pin_constant(_mut_tie_high))
    assert not (pin_topk(_mut_unstable_zero) and pin_constant(_mut_unstable_zero))
