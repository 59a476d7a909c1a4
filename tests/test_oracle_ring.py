"""Pins of the ring-attention oracle: a two-key closed form (fixes the scale
and which operand is transposed), the Q = 0 and equal-keys limits (uniform
weights), a dominant key (hard attention), constant values, invariance under a
joint permutation of keys and values, brute force with exact sums on a tiny
case, the log-sum-exp merge of per-shard partial results in ring order, and
the ring order itself."""
import math

import numpy as np

import oracle.ring_attn as ora
from oracle.numerics import bf16_to_f64, f64_to_bf16_bits
import workloads as wl


def _bf(x):
    return f64_to_bf16_bits(np.asarray(x, np.float64))


def test_ring_order():
    assert ora.ring_order(1) == [0]
    assert ora.ring_order(4) == [0, 3, 2, 1]
    assert sorted(ora.ring_order(8)) == list(range(8))


def test_two_keys_closed_form():
    # one query, two keys in two shards: weight of key 1 is the logistic of
    # (q.k1 - q.k0) / sqrt(D)
    D = 4
    q = np.array([[[1.0, 2.0, 0.5, -1.0]]])
    k0 = np.array([[[0.5, 0.0, 1.0, 0.0]]])
    k1 = np.array([[[1.0, 1.0, 0.0, 2.0]]])
    v0 = np.array([[[1.0, 0.0, -2.0, 4.0]]])
    v1 = np.array([[[0.0, 3.0, 1.0, -1.0]]])
    O, _ = ora.ring_attention(_bf(q), [_bf(k0), _bf(k1)], [_bf(v0), _bf(v1)])
    d = (q[0, 0] @ k1[0, 0] - q[0, 0] @ k0[0, 0]) / math.sqrt(D)    # (1 + 2 - 2 - 0.5) / 2
    w1 = 1.0 / (1.0 + math.exp(-d))
    assert np.allclose(O[0, 0], (1 - w1) * v0[0, 0] + w1 * v1[0, 0], rtol=0, atol=1e-15)


def test_zero_queries_average_all_values():
    w = wl.make_ring(2, 16, 8, 3, seed=61)
    Q0 = np.zeros_like(w.Q)
    O, _ = ora.ring_attention(Q0, w.K, w.V)
    mean = np.concatenate([bf16_to_f64(v) for v in w.V], axis=1).mean(axis=1)
    for h in range(2):
        assert np.allclose(O[h], mean[h][None, :], rtol=0, atol=1e-14)


def test_equal_keys_average_all_values():
    w = wl.make_ring(1, 8, 16, 4, seed=62)
    K = [np.broadcast_to(w.K[0][:, :1, :], w.K[0].shape).copy() for _ in range(4)]
    O, _ = ora.ring_attention(w.Q, K, w.V)
    mean = np.concatenate([bf16_to_f64(v) for v in w.V], axis=1).mean(axis=1)
    assert np.allclose(O[0], mean[0][None, :], rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    # q = 8 e0, one key 8 e0 (score 64 / sqrt(D) = 16 above the others, which
    # are orthogonal): the output is that key's value within exp(-16) * range
    H, S, D, R = 1, 4, 16, 3
    w = wl.make_ring(H, S, D, R, seed=63)
    q = np.zeros((H, S, D)); q[:, :, 0] = 8.0
    K = [np.zeros((H, S, D)) for _ in range(R)]
    for r in range(R):
        K[r][0, :, 1] = 1.0
    K[2][0, 3, :] = 0.0
    K[2][0, 3, 0] = 8.0
    O, _ = ora.ring_attention(_bf(q), [_bf(k) for k in K], w.V)
    v = bf16_to_f64(w.V[2][0, 3])
    spread = max(np.abs(bf16_to_f64(x)).max() for x in w.V)
    assert np.abs(O[0] - v[None, :]).max() <= 2 * R * S * math.exp(-16.0) * spread


def test_constant_values_give_that_constant():
    w = wl.make_ring(2, 8, 8, 2, seed=64)
    V = [np.full_like(v, _bf(np.array(1.5))) for v in w.V]
    O, _ = ora.ring_attention(w.Q, w.K, V)
    assert np.allclose(O, 1.5, rtol=0, atol=1e-14)


def test_joint_key_value_permutation_is_invariant():
    w = wl.make_ring(2, 8, 16, 3, seed=65)
    O, _ = ora.ring_attention(w.Q, w.K, w.V)
    K = np.concatenate(w.K, axis=1)
    V = np.concatenate(w.V, axis=1)
    p = np.random.default_rng(0).permutation(K.shape[1])
    Ks = np.split(K[:, p], 3, axis=1)
    Vs = np.split(V[:, p], 3, axis=1)
    O2, _ = ora.ring_attention(w.Q, Ks, Vs)
    assert np.allclose(O, O2, rtol=0, atol=1e-13)
    # shuffling values alone (not keys) changes the result
    Vb = np.split(V[:, p], 3, axis=1)
    O3, _ = ora.ring_attention(w.Q, w.K, Vb)
    assert np.abs(O - O3).max() > 1e-3


def test_brute_force_exact_sums():
    w = wl.make_ring(2, 3, 4, 2, seed=66)
    O, Ob = ora.ring_attention(w.Q, w.K, w.V)
    q = bf16_to_f64(w.Q)
    K = [bf16_to_f64(k) for k in w.K]
    V = [bf16_to_f64(v) for v in w.V]
    for h in range(2):
        for i in range(3):
            keys = [(K[r][h, j], V[r][h, j]) for r in range(2) for j in range(3)]
            sc = [math.fsum(q[h, i, d] * k[d] for d in range(4)) / 2.0 for k, _ in keys]
            e = [math.exp(x) for x in sc]
            den = math.fsum(e)
            for d in range(4):
                ref = math.fsum(e[j] * keys[j][1][d] for j in range(len(keys))) / den
                assert abs(O[h, i, d] - ref) <= 1e-14
    assert np.array_equal(Ob, f64_to_bf16_bits(O))


def test_shard_merge_in_ring_order_matches():
    # each step's partial result (row max m, row sum l, unnormalised output o)
    # merged by rescaling with exp(m_old - m_new) gives the one-shot softmax
    w = wl.make_ring(2, 8, 16, 4, seed=67)
    O, _ = ora.ring_attention(w.Q, w.K, w.V)
    q = bf16_to_f64(w.Q)
    m = np.full(q.shape[:2], -np.inf)
    l = np.zeros(q.shape[:2])
    o = np.zeros(q.shape)
    for r in ora.ring_order(4):
        s = np.einsum("hid,hjd->hij", q, bf16_to_f64(w.K[r])) / 4.0
        mn = np.maximum(m, s.max(axis=2))
        c = np.exp(m - mn)
        p = np.exp(s - mn[:, :, None])
        l = l * c + p.sum(axis=2)
        o = o * c[:, :, None] + np.einsum("hij,hjd->hid", p, bf16_to_f64(w.V[r]))
        m = mn
    assert np.allclose(O, o / l[:, :, None], rtol=1e-13, atol=1e-14)


def test_rows_helper_matches_full():
    w = wl.make_ring(3, 16, 8, 2, seed=68)
    O, _ = ora.ring_attention(w.Q, w.K, w.V)
    rows = [0, 5, 15]
    assert np.allclose(ora.ring_attention_rows(w.Q, w.K, w.V, 2, rows), O[2, rows], rtol=0, atol=1e-14)


def test_one_rank_is_plain_attention_and_f32_output():
    w = wl.make_ring(1, 6, 4, 1, seed=69)
    O, O32 = ora.ring_attention(w.Q, w.K, w.V, "f32")
    q, k, v = (bf16_to_f64(x)[0] for x in (w.Q, w.K[0], w.V[0]))
    s = q @ k.T / 2.0
    p = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    assert np.allclose(O[0], p @ v, rtol=1e-13, atol=1e-15)
    assert O32.dtype == np.float32
