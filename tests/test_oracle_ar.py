"""Pins of the GEMM -> AllReduce oracle: brute force with exact sums, the
all-reduce as reduce-scatter followed by all-gather, integer inputs against
integer arithmetic, and the degenerate cases (one rank, zero A)."""
import math

import numpy as np

import oracle.gemm_ar as oar
import oracle.gemm_rs as orc
from oracle.numerics import bf16_to_f64
import workloads as wl


def test_fsum_brute_force_and_every_rank_gets_the_sum():
    w = wl.make_rs(24, 40, 32, 3, seed=51)
    S, outs = oar.gemm_ar(w.A, w.B, w.partials, w.R)
    a, b = bf16_to_f64(w.A), bf16_to_f64(w.B)
    for i in range(w.M):
        for j in range(w.N):
            terms = [a[i, k] * b[k, j] for k in range(w.K)] + [float(P[i, j]) for P in w.partials]
            assert abs(S[i, j] - math.fsum(terms)) <= 1e-13 * sum(abs(t) for t in terms) + 1e-300
    assert len(outs) == w.R
    assert all(np.array_equal(o, S.astype(np.float32)) for o in outs)


def test_all_reduce_is_reduce_scatter_then_all_gather():
    w = wl.make_rs(64, 40, 24, 8, seed=52, dist="int")
    S, outs = oar.gemm_ar(w.A, w.B, w.partials, w.R)
    _, blocks, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    assert np.array_equal(np.vstack(blocks), S)


def test_integer_inputs_match_integer_arithmetic():
    w = wl.make_rs(40, 48, 16, 4, seed=53, dist="int")
    S, outs = oar.gemm_ar(w.A, w.B, w.partials, w.R, "bf16")
    a = bf16_to_f64(w.A).astype(np.int64)
    b = bf16_to_f64(w.B).astype(np.int64)
    ref = a @ b
    for P in w.partials:
        ref = ref + P.astype(np.int64)
    assert np.array_equal(S, ref.astype(np.float64))


def test_one_rank_is_the_plain_gemm():
    w = wl.make_rs(30, 32, 16, 1, seed=54)
    S, outs = oar.gemm_ar(w.A, w.B, w.partials, 1)
    assert w.partials == []
    C = np.array([[math.fsum(bf16_to_f64(w.A)[i, k] * bf16_to_f64(w.B)[k, j] for k in range(32))
                   for j in range(16)] for i in range(30)])
    assert np.allclose(S, C, rtol=1e-14, atol=1e-12)
    assert len(outs) == 1


def test_zero_A_gives_sum_of_partials_for_ragged_M():
    # M = 45 is not a multiple of R = 4: allowed for the all-reduce
    w = wl.make_rs(45 * 4, 32, 16, 4, seed=55, dist="int")
    A0 = np.zeros((45, 32), w.A.dtype)
    parts = [P[:45] for P in w.partials]
    S, outs = oar.gemm_ar(A0, w.B, parts, 4)
    assert np.array_equal(S, sum(P.astype(np.float64) for P in parts))
