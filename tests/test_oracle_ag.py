"""Pins of the AllGather -> GEMM oracle against brute force, closed forms,
exact integer arithmetic and arrival-order independence.  The mutation tests
plant plausible mistakes in copies of the oracle and check a pin catches each."""
import math

import numpy as np
import pytest

import oracle.ag_gemm as og
from oracle.numerics import bf16_to_f64
from oracle.schedule import ScheduleError
import workloads as wl

ONE = np.uint16(0x3F80)


def _fsum_C(shards, B):
    A = np.vstack(shards)
    a, b = bf16_to_f64(A), bf16_to_f64(B)
    M, K = a.shape
    N = b.shape[1]
    C = np.empty((M, N))
    S = np.empty((M, N))
    for i in range(M):
        prods = a[i][:, None] * b            # exact: 8-bit x 8-bit significands
        for j in range(N):
            C[i, j] = math.fsum(prods[:, j])
        S[i] = np.abs(prods).sum(0)
    return C, S


# ---- pin functions (take the function under test so mutants can be checked) ----
def pin_fsum(fn, w):
    C64, _ = fn(w.shards, w.B, "f32")
    ref, S = _fsum_C(w.shards, w.B)
    return np.all(np.abs(C64 - ref) <= 1e-13 * S + 1e-300)


def pin_identity(fn, seed=3):
    # B = I: the product IS the gathered A, shard r at rows [r*m, (r+1)*m).
    w = wl.make_ag(5, 8, 24, 24, seed=seed, dist="uniform")
    B = np.where(np.eye(24, dtype=bool), ONE, np.uint16(0))
    C64, _ = fn(w.shards, B, "f32", order=w.order[::-1].copy(), unit_rows=8)
    want = np.stack([bf16_to_f64(w.shards[i // 8][i % 8]) for i in range(40)])
    return np.array_equal(C64, want)


def pin_onehot(fn, seed=4):
    # A rows are one-hot at column p(i): C row i is B row p(i).
    rng = np.random.default_rng(seed)
    K, N, R, m = 16, 16, 2, 6
    p = rng.integers(0, K, size=R * m)
    A = np.zeros((R * m, K), np.uint16)
    A[np.arange(R * m), p] = ONE
    B = wl.make_ag(1, 1, K, N, seed=seed, dist="uniform").B
    C64, _ = fn([A[:m], A[m:]], B, "f32")
    return np.array_equal(C64, bf16_to_f64(B)[p])


def pin_integer(fn, seed=5):
    w = wl.make_ag(3, 7, 40, 9, seed=seed, dist="int")
    C64, _ = fn(w.shards, w.B, "f32")
    Ai = np.vstack([bf16_to_f64(s) for s in w.shards]).astype(np.int64)
    Bi = bf16_to_f64(w.B).astype(np.int64)
    ref = np.einsum("ik,kj->ij", Ai, Bi)    # exact integer arithmetic, other path
    return np.array_equal(C64, ref.astype(np.float64))


# ---- the pins on the oracle ----
def test_fsum_brute_force_tiny_config():
    w = wl.CONFIGS["tiny_ag"]["make"]()
    assert (w.M, w.K, w.N) == (256, 128, 96)
    assert pin_fsum(og.ag_gemm, w)


def test_identity_B_gives_gathered_A_in_rank_order():
    assert pin_identity(og.ag_gemm)


def test_onehot_rows_select_B_rows():
    assert pin_onehot(og.ag_gemm)


def test_integer_inputs_are_exact():
    assert pin_integer(og.ag_gemm)


def test_result_independent_of_arrival_schedule():
    w = wl.make_ag(4, 16, 32, 24, seed=7, unit_rows=8)
    outs = [og.ag_gemm(w.shards, w.B, "bf16", order=o, unit_rows=8)[1]
            for o in (np.arange(8), np.arange(8)[::-1].copy(), w.order)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])


def test_rows_helper_matches_full():
    w = wl.make_ag(3, 10, 32, 17, seed=8)
    C64, _ = og.ag_gemm(w.shards, w.B)
    rows = [0, 9, 10, 29, 17]
    assert np.array_equal(og.ag_gemm_rows(w.shards, w.B, rows), C64[rows])


def test_bf16_output_is_rounded_once():
    w = wl.make_ag(2, 8, 16, 8, seed=9)
    C64, C = og.ag_gemm(w.shards, w.B, "bf16")
    assert C.dtype == np.uint16
    err = np.abs(bf16_to_f64(C) - C64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(C64))[1] - 8)
    assert np.all(err <= 0.5 * ulp)


@pytest.mark.parametrize("bad", [np.array([0, 0, 1, 2]), np.array([0, 1, 2]), np.array([0, 1, 2, 4])])
def test_schedule_validation_rejects(bad):
    w = wl.make_ag(4, 8, 16, 8, seed=1)
    with pytest.raises(ScheduleError):
        og.ag_gemm(w.shards, w.B, order=bad, unit_rows=8)


def test_tile_units_brute_force():
    for M, BM, ur in [(256, 64, 64), (8192, 256, 128), (128, 256, 16), (100, 32, 10)]:
        for t in range((M + BM - 1) // BM):
            rows = range(t * BM, min(M, (t + 1) * BM))
            units = sorted({r // ur for r in rows})
            assert og.tile_units(t, BM, ur, M) == (units[0], units[-1])
            assert units == list(range(units[0], units[-1] + 1))


# ---- mutation tests: each planted mistake must be caught by some pin ----
def _mut_arrival_order(shards, B, out_dtype="bf16", order=None, delay_ns=None, unit_rows=None):
    if order is not None:
        m = unit_rows or shards[0].shape[0]
        A = np.vstack(shards)
        A = np.vstack([A[c * m:(c + 1) * m] for c in order])
        C = bf16_to_f64(A) @ bf16_to_f64(B)
        return C, C
    return og.ag_gemm(shards, B, out_dtype)


def _mut_transposed_B(shards, B, out_dtype="bf16", **kw):
    C = bf16_to_f64(np.vstack(shards)) @ bf16_to_f64(B).T if B.shape[0] == B.shape[1] else None
    return (C, C) if C is not None else og.ag_gemm(shards, B, out_dtype)


def _mut_dropped_term(shards, B, out_dtype="bf16", **kw):
    a = bf16_to_f64(np.vstack(shards))
    b = bf16_to_f64(B)
    C = a[:, :-1] @ b[:-1]
    return C, C


def test_mutants_are_caught():
    w = wl.CONFIGS["tiny_ag"]["make"]()
    assert not pin_identity(_mut_arrival_order)
    assert not pin_onehot(_mut_transposed_B)
    assert not (pin_fsum(_mut_dropped_term, w) and pin_integer(_mut_dropped_term))
