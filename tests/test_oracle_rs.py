"""Pins of the GEMM -> ReduceScatter oracle: brute force, reduce-scatter over
all owners equals the all-reduce computed by a separate path, and the two
degenerate cases (no partials, zero A)."""
import math

import numpy as np

import oracle.gemm_rs as orc
from oracle.numerics import bf16_to_f64
import workloads as wl


def pin_fsum(fn, w):
    S, blocks, _ = fn(w.A, w.B, w.partials, w.R)
    a, b = bf16_to_f64(w.A), bf16_to_f64(w.B)
    ok = True
    for i in range(w.M):
        prods = a[i][:, None] * b
        for j in range(w.N):
            terms = list(prods[:, j]) + [float(P[i, j]) for P in w.partials]
            ref = math.fsum(terms)
            ok &= abs(S[i, j] - ref) <= 1e-13 * sum(abs(t) for t in terms) + 1e-300
    return bool(ok)


def pin_slice_then_sum(fn, w):
    """Owner blocks equal each owner's rows reduced on their own (other path)."""
    S, blocks, _ = fn(w.A, w.B, w.partials, w.R)
    mb = w.M // w.R
    ok = np.array_equal(np.vstack(blocks), S)
    a, b = bf16_to_f64(w.A), bf16_to_f64(w.B)
    for r in range(w.R):
        rows = slice(r * mb, (r + 1) * mb)
        acc = np.einsum("ik,kj->ij", a[rows].astype(np.int64), b.astype(np.int64)).astype(np.float64)
        for P in w.partials:
            acc = acc + P[rows].astype(np.float64)
        ok &= np.array_equal(blocks[r], acc)
    return bool(ok)


def test_fsum_brute_force():
    w = wl.make_rs(32, 48, 40, 4, seed=11)
    assert pin_fsum(orc.gemm_rs, w)


def test_reduce_scatter_over_owners_is_all_reduce():
    w = wl.make_rs(64, 40, 24, 8, seed=12, dist="int")
    assert pin_slice_then_sum(orc.gemm_rs, w)


def test_no_partials_reduces_to_sliced_gemm():
    w = wl.make_rs(48, 32, 16, 4, seed=13, dist="int")
    S, blocks, _ = orc.gemm_rs(w.A, w.B, [np.zeros_like(P) for P in w.partials], w.R)
    C = bf16_to_f64(w.A) @ bf16_to_f64(w.B)
    assert all(np.array_equal(blocks[r], C[r * 12:(r + 1) * 12]) for r in range(4))


def test_zero_A_gives_sum_of_partials():
    w = wl.make_rs(48, 32, 16, 4, seed=14, dist="int")
    A0 = np.zeros_like(w.A)
    S, _, outs = orc.gemm_rs(A0, w.B, w.partials, w.R)
    ref = np.zeros_like(S)
    for P in w.partials:
        ref += P
    assert np.array_equal(S, ref)
    assert np.array_equal(np.vstack(outs), ref.astype(np.float32))


def test_rows_helper_matches_full():
    w = wl.make_rs(40, 24, 16, 4, seed=15)
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    rows = [0, 5, 39, 20]
    assert np.allclose(orc.gemm_rs_rows(w.A, w.B, w.partials, rows), S[rows], rtol=0, atol=1e-12)


def test_owner_map_brute_force():
    M, R = 8192, 8
    for BM in (128, 256, 1024):
        for t in range(M // BM):
            owners = {r * R // M for r in range(t * BM, (t + 1) * BM)}
            assert owners == {orc.tile_owner(t, BM, M, R)}


# ---- mutants ----
def _mut_drop_partial(A, B, partials, R, out_dtype="f32"):
    return orc.gemm_rs(A, B, partials[:-1], R, out_dtype)


def _mut_interleaved_owner(A, B, partials, R, out_dtype="f32"):
    S, blocks, outs = orc.gemm_rs(A, B, partials, R, out_dtype)
    blocks = [S[r::R] for r in range(R)]
    return S, blocks, blocks


def test_mutants_are_caught():
    w = wl.make_rs(32, 16, 8, 4, seed=16, dist="int")
    assert pin_slice_then_sum(orc.gemm_rs, w)
    assert not pin_slice_then_sum(_mut_drop_partial, w)
    assert not pin_slice_then_sum(_mut_interleaved_owner, w)
