"""Pins of the MoE combine oracle: the gate weights (a softmax over the k
selected logits: sum 1, descending with the logits, uniform for equal logits,
1 for k = 1), brute force with exact sums and a linear search for each pair's
dispatch position, and the end-to-end closed form: combining the dispatch +
grouped-GEMM outputs (local experts) and directly computed peer outputs gives
sum_j g_j * X[t] @ W[e_j] for every token, with integer inputs exactly."""
import math

import numpy as np

import oracle.moe as om
import oracle.moe_combine as oc
from oracle.numerics import bf16_to_f64, f64_to_bf16_bits
import workloads as wl


def test_gate_weights():
    w = wl.make_moe(64, 16, 32, 6, 8, 8, seed=41, block_tokens=16)
    topk = om.route_topk(w.logits, w.k)
    g = oc.gate_weights(w.logits, topk)
    assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(g, axis=1) <= 1e-18)              # slots are in descending logit order
    eq = np.zeros((4, 8), np.float32)
    assert np.allclose(oc.gate_weights(eq, om.route_topk(eq, 4)), 0.25, rtol=0, atol=1e-16)
    assert np.array_equal(oc.gate_weights(w.logits, topk[:, :1]), np.ones((64, 1)))
    # two slots: the weight of slot 0 is the logistic of the logit difference
    t2 = topk[:, :2]
    l = np.take_along_axis(w.logits.astype(np.float64), t2, axis=1)
    assert np.allclose(oc.gate_weights(w.logits, t2)[:, 0], 1 / (1 + np.exp(l[:, 1] - l[:, 0])), rtol=1e-14, atol=0)


def test_brute_force_with_linear_search():
    w = wl.make_moe(16, 8, 12, 3, 4, 8, seed=42, expert_begin=5, block_tokens=8)
    Yl, Yp = wl.moe_combine_inputs(w, seed=1)
    topk = om.route_topk(w.logits, w.k)
    counts, offsets, perm = om.dispatch(topk, w.E)
    out, out_bf = oc.moe_combine(Yl, Yp, w.logits, topk, perm, offsets, 5, 4)
    lo, hi = int(offsets[5]), int(offsets[9])
    yl, yp = bf16_to_f64(Yl), bf16_to_f64(Yp)
    for t in range(w.T):
        ls = [float(w.logits[t, e]) for e in topk[t]]
        ex = [math.exp(x - max(ls)) for x in ls]
        den = math.fsum(ex)
        for f in range(w.F):
            terms = []
            for j in range(w.k):
                p = [i for i in range(len(perm)) if perm[i] == t * w.k + j]
                assert len(p) == 1
                p = p[0]
                y = yl[p - lo, f] if lo <= p < hi else yp[p, f]
                terms.append(ex[j] / den * y)
            assert abs(out[t, f] - math.fsum(terms)) <= 1e-14 * (1 + sum(abs(x) for x in terms))
    assert np.array_equal(out_bf, f64_to_bf16_bits(out))


def _direct(X, Wall, logits, topk):
    g = oc.gate_weights(logits, topk)
    x = bf16_to_f64(X)
    out = np.zeros((x.shape[0], Wall[0].shape[1]))
    for t in range(x.shape[0]):
        for j, e in enumerate(topk[t]):
            out[t] += g[t, j] * (x[t] @ bf16_to_f64(Wall[e]))
    return out


def test_dispatch_gemm_then_combine_is_the_weighted_expert_sum():
    # integer inputs: every expert output is a small integer, exact in bf16
    T, H, E, k, F, eb, L = 48, 16, 10, 3, 8, 3, 4
    w = wl.make_moe(T, H, E, k, L, F, seed=43, expert_begin=eb, block_tokens=16, dist="int")
    rng = np.random.default_rng(44)
    Wall = [f64_to_bf16_bits(rng.integers(-1, 2, size=(H, F)).astype(np.float64)) for _ in range(E)]
    Wall[eb:eb + L] = w.W
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, k, eb, "bf16")
    assert np.max(np.abs(ref["Y64"])) <= 256                     # exact in bf16
    topk, offsets, perm = ref["topk"], ref["offsets"], ref["perm"]
    # peer outputs: one row per dispatch position, computed pair by pair
    x = bf16_to_f64(w.X)
    Yp = np.zeros((T * k, F))
    for p, pair in enumerate(perm):
        t, j = divmod(int(pair), k)
        Yp[p] = x[t] @ bf16_to_f64(Wall[topk[t, j]])
    out, _ = oc.moe_combine(ref["Y"], f64_to_bf16_bits(Yp), w.logits, topk, perm, offsets, eb, L)
    assert np.allclose(out, _direct(w.X, Wall, w.logits, topk), rtol=1e-13, atol=1e-12)
    # the local rows matter: taking every row from the peers' buffer differs
    bad, _ = oc.moe_combine(ref["Y"], f64_to_bf16_bits(Yp * 0 + 1.0), w.logits, topk, perm, offsets, eb, L)
    assert not np.allclose(bad, out)


def test_all_experts_local_needs_no_peer_rows():
    w = wl.make_moe(32, 16, 8, 2, 8, 8, seed=45, block_tokens=16, dist="int")
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "bf16")
    nan_peer = np.full((w.T * w.k, w.F), 0x7fc0, np.uint16)       # never read
    out, _ = oc.moe_combine(ref["Y"], nan_peer, w.logits, ref["topk"], ref["perm"], ref["offsets"], 0, 8)
    assert np.all(np.isfinite(out))
    assert np.allclose(out, _direct(w.X, w.W, w.logits, ref["topk"]), rtol=1e-13, atol=1e-12)
