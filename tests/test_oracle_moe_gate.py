"""Pins of the MoE gate GEMM oracle: brute force with math.fsum, closed forms
(identity gate, one-hot tokens), exact integer arithmetic by a separate path,
the float32 rounding of the result, and a planted mistake that a pin catches."""
import math

import numpy as np

import oracle.moe_gate as og
from oracle.numerics import bf16_to_f64
import workloads as wl
from workloads import f32_to_bf16_bits


def _small(seed=1, dist="normal"):
    w = wl.make_moe(48, 40, 24, 3, 6, 16, seed=seed, block_tokens=16)
    return w, wl.moe_gate_weights(w, seed=seed, dist=dist)


def test_fsum_brute_force():
    w, Wg = _small()
    L64, L32 = og.gate_logits(w.X, Wg)
    x, g = bf16_to_f64(w.X), bf16_to_f64(Wg)
    for t in range(w.X.shape[0]):
        for e in range(Wg.shape[1]):
            terms = x[t] * g[:, e]                    # exact products of bf16 values
            ref = math.fsum(terms.tolist())
            assert abs(L64[t, e] - ref) <= 4 * np.spacing(np.abs(terms).sum() + 1e-300)
    assert L32.dtype == np.float32 and np.array_equal(L32, L64.astype(np.float32))


def test_identity_gate_gives_the_tokens():
    # H = E and W_gate = I: each logit is the token's own entry, exactly
    w = wl.make_moe(16, 24, 24, 2, 4, 8, seed=3, block_tokens=8)
    I = f32_to_bf16_bits(np.eye(24, dtype=np.float32))
    L64, L32 = og.gate_logits(w.X, I)
    assert np.array_equal(L64, bf16_to_f64(w.X))


def test_one_hot_tokens_give_gate_rows():
    w, Wg = _small(seed=4)
    X = np.zeros_like(w.X)
    for t in range(X.shape[0]):
        X[t, t % X.shape[1]] = f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    L64, _ = og.gate_logits(X, Wg)
    g = bf16_to_f64(Wg)
    for t in range(X.shape[0]):
        assert np.array_equal(L64[t], g[t % X.shape[1]])


def test_integer_inputs_exact_by_int64():
    w, Wg = _small(seed=5, dist="int")
    Xi = np.rint(bf16_to_f64(w.X)).astype(np.int64)      # the workload's X is normal: use an integer copy
    Xb = f32_to_bf16_bits(np.clip(Xi, -2, 2).astype(np.float32))
    L64, L32 = og.gate_logits(Xb, Wg)
    ref = bf16_to_f64(Xb).astype(np.int64) @ bf16_to_f64(Wg).astype(np.int64)
    assert np.array_equal(L64, ref.astype(np.float64))
    assert np.array_equal(L32, ref.astype(np.float32))


def test_planted_transposed_gate_is_caught():
    # a plausible mistake, X @ W_gate^T on a square gate, fails the brute force
    w = wl.make_moe(8, 16, 16, 2, 4, 8, seed=6, block_tokens=8)
    Wg = wl.moe_gate_weights(w, seed=6)
    wrong = bf16_to_f64(w.X) @ bf16_to_f64(Wg).T
    right, _ = og.gate_logits(w.X, Wg)
    assert not np.allclose(wrong, right)


def test_gate_weights_draw_leaves_the_workload_unchanged():
    a = wl.make_moe(48, 40, 24, 3, 6, 16, seed=7, block_tokens=16)
    Wg = wl.moe_gate_weights(a, seed=7)
    b = wl.make_moe(48, 40, 24, 3, 6, 16, seed=7, block_tokens=16)
    assert np.array_equal(a.X, b.X) and np.array_equal(a.logits, b.logits)
    assert Wg.shape == (40, 24) and Wg.dtype == np.uint16
    v = bf16_to_f64(Wg)
    assert abs(v.var() * 40 - 1.0) < 0.35                 # N(0, 1/H)
