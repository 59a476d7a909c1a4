"""Pins of the GEMM -> ReduceScatter oracle: brute force, reduce-scatter over
all owners equals the all-reduce computed by a separate path, and the two
degenerate cases (no partials, zero A)."""
import math

import numpy as np
import pytest

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


def test_partial_units_are_peer_major_row_blocks():
    # M = 8 rows in blocks of 2, R = 3 (peers 1 and 2): 8 units, peer-major
    M, R, ur = 8, 3, 2
    assert orc.partial_units(M, R, ur) == 8
    ids = [[orc.unit_of(p, r, M, ur) for r in range(M)] for p in (1, 2)]
    assert ids == [[0, 0, 1, 1, 2, 2, 3, 3], [4, 4, 5, 5, 6, 6, 7, 7]]
    # every (peer, row) lands in exactly one unit and every unit is hit
    assert sorted({u for row in ids for u in row}) == list(range(8))


def test_rs_schedule_validated_and_ignored():
    from oracle.schedule import ScheduleError
    w = wl.make_rs(64, 16, 24, 4, seed=5, unit_rows=16, max_delay_ns=20000)
    assert w.order.shape == (3 * 4,) and sorted(w.order.tolist()) == list(range(12))
    assert np.all(w.delay_ns <= 20000)
    S0, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    S1, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R, order=w.order, delay_ns=w.delay_ns, unit_rows=16)
    assert np.array_equal(S0, S1)
    with pytest.raises(ScheduleError):
        orc.gemm_rs(w.A, w.B, w.partials, w.R, order=w.order[:-1], unit_rows=16)
    bad = w.order.copy()
    bad[0] = bad[1]
    with pytest.raises(ScheduleError):
        orc.gemm_rs(w.A, w.B, w.partials, w.R, order=bad, unit_rows=16)
    with pytest.raises(ScheduleError):
        orc.partial_units(64, 4, 24)


def test_rs_schedule_draw_leaves_the_tensors_unchanged():
    a = wl.make_rs(64, 16, 24, 4, seed=5)
    b = wl.make_rs(64, 16, 24, 4, seed=5, unit_rows=16)
    assert np.array_equal(a.A, b.A) and np.array_equal(a.B, b.B)
    assert all(np.array_equal(x, y) for x, y in zip(a.partials, b.partials))
