"""Seeded random shapes and launch options for every operation, checked
against the float64 oracle.  The GEMM paths (AllGather + GEMM, GEMM +
ReduceScatter / AllReduce, MoE dispatch + grouped GEMM, the gate) take
integer-valued inputs with float32 outputs, where every partial sum is exact,
so their outputs must match bit for bit whatever the tile, role split, grid,
queue order, copy item size or arrival schedule; the combine and ring
attention (softmax weights) are held to the floating-point tolerance.  The
cases come from fixed seeds, so every run draws the same ones; each case is
printed before it runs."""
import numpy as np
import pytest
import torch

import oracle.ag_gemm as og
import oracle.gemm_ar as oar
import oracle.gemm_rs as ors
import oracle.moe as om
import oracle.moe_combine as oc
import oracle.moe_gate as ogate
import oracle.ring_attn as ora
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _divisors(n):
    return [d for d in range(1, n + 1) if n % d == 0]


# ------------------------------------------------------------ AllGather + GEMM
def _ag_cases(seed=2024):
    # every tile id (0 = the per-shape default) at least once; a tile with a
    # K or M condition usually gets a shape it supports, now and then one it
    # must reject
    rng = np.random.default_rng(seed)
    out = []
    for i, tile in enumerate(2 * [0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 0, 5, 10, 11, 11, 9]):
        R = int(rng.integers(1, 9))
        fits = rng.random() < 0.8
        m = int(rng.integers(1, 128 // R + 1)) if tile == 11 and fits else int(rng.integers(1, 160))
        M = R * m
        ks = [128, 256, 384, 512, 640, 1024] if fits and tile in (5, 6, 7, 8, 10, 11) else \
             [256, 512, 768, 1024] if fits and tile == 9 else [8, 64, 128, 200, 256, 384, 512, 640, 1024]
        K = int(rng.choice(ks))
        N = 8 * int(rng.integers(1, 80))
        unit_rows = int(rng.choice([d for d in _divisors(M) if M // d <= 256]))
        lau = dict(tile=tile, grid=int(rng.choice([0, 0, 3, 17, 100])), n_copy=int(rng.choice([0, 0, 1, 5])),
                   mode=int(rng.choice([0, 0, 0, 1])), queue_mode=int(rng.choice([0, 1])),
                   copy_kib=int(rng.choice([0, 0, 1, 16])))
        out.append((i, R, m, K, N, unit_rows, int(rng.integers(0, 3000)), lau))
    return out


def _ag_tile_ok(tile, M, K):
    if tile in (5, 6, 7, 8, 10):
        return K % 128 == 0
    if tile == 9:
        return K % 256 == 0
    if tile == 11:
        return M <= 128 and K % 128 == 0
    return True


@pytest.mark.parametrize("case", _ag_cases(), ids=lambda c: f"ag{c[0]}")
def test_fuzz_ag(gpu, case):
    from tile_pipelined_gemm_amd.harness import AgProblem, to_numpy
    i, R, m, K, N, unit_rows, delay, lau = case
    print(f"AG case {i}: R={R} m_shard={m} K={K} N={N} unit_rows={unit_rows} max_delay_ns={delay} launch={lau}",
          flush=True)
    w = wl.make_ag(R, m, K, N, seed=100 + i, dist="int", unit_rows=unit_rows, max_delay_ns=delay, out_dtype="f32")
    prob = AgProblem(w)
    prob.Ag.fill_(float("nan"))
    rc = prob.run(launch=gpu.make_launch(**lau), check=False)
    if not _ag_tile_ok(lau["tile"], w.M, K):
        assert rc == gpu.MK_ERR_UNSUPPORTED
        return
    assert rc == gpu.MK_OK, gpu.load().mk_last_error()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)
    assert np.array_equal(to_numpy(prob.Ag), og.gather(w.shards))


# ------------------------------------------------- GEMM + ReduceScatter / AllReduce
def _rs_cases(seed=2025):
    rng = np.random.default_rng(seed)
    out = []
    for i, tile in enumerate(2 * [0, 2, 3, 4, 5, 6, 7, 8, 0, 5, 1, 9]):
        R = int(rng.integers(2, 9))
        mb = int(rng.choice([128, 256, 384]))
        K = int(rng.choice([128, 256, 512] if tile in (5, 6, 7, 8) and rng.random() < 0.8 else [8, 128, 136, 256, 512]))
        N = 8 * int(rng.integers(1, 64))
        arrival = bool(rng.integers(0, 2))
        landing = arrival and bool(rng.integers(0, 2))
        unit_rows = int(rng.choice([d for d in _divisors(mb) if (R - 1) * (R * mb // d) <= 256 and d % 8 == 0]))
        lau = dict(grid=int(rng.choice([0, 0, 7, 64])), n_reduce=int(rng.choice([0, 0, -1, 4])),
                   mode=int(rng.choice([0, 0, 1])), tile=tile,
                   copy_kib=int(rng.choice([0, 0, 4])))
        out.append((i, R, mb, K, N, arrival, landing, unit_rows, lau))
    return out


def _rs_tile_ok(tile, mb, K, all_reduce):
    if tile in (1, 9, 10, 11):      # not built for this operation
        return False
    if tile in (5, 6, 7, 8) and K % 128:
        return False
    bm = 256 if tile in (1, 3, 5, 7) else 128
    return all_reduce or tile == 0 or mb % bm == 0


@pytest.mark.parametrize("case", _rs_cases(), ids=lambda c: f"rs{c[0]}")
def test_fuzz_rs_and_ar(gpu, case):
    from tile_pipelined_gemm_amd.harness import RsProblem, ArProblem
    i, R, mb, K, N, arrival, landing, unit_rows, lau = case
    M = R * mb
    print(f"RS/AR case {i}: M={M} K={K} N={N} R={R} arrival={arrival} landing={landing} unit_rows={unit_rows} "
          f"launch={lau}", flush=True)
    w = wl.make_rs(M, K, N, R, seed=200 + i, dist="int", out_dtype="f32",
                   unit_rows=unit_rows if arrival else None, max_delay_ns=2000 if arrival else 0)
    S64, _, blocks = ors.gemm_rs(w.A, w.B, w.partials, R, "f32")
    _, ar_outs = oar.gemm_ar(w.A, w.B, w.partials, R, "f32")
    for P in (RsProblem(w, landing=landing), ArProblem(w, landing=landing)):
        ar = isinstance(P, ArProblem)
        for o in P.out:
            o.fill_(float("nan"))
        if landing:
            for b in P.landing:
                b.fill_(float("nan"))
        rc = P.run(launch=gpu.make_launch(**lau), check=False)
        if not _rs_tile_ok(lau["tile"], mb, K, ar):
            assert rc == gpu.MK_ERR_UNSUPPORTED, ("AR" if ar else "RS")
            continue
        assert rc == gpu.MK_OK, gpu.load().mk_last_error()
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(P.ws) == gpu.MK_OK
        if ar:
            for r, o in enumerate(P.outputs()):
                assert np.array_equal(o, ar_outs[r]), f"AR output {r}"
        else:
            assert np.array_equal(P.output(), np.vstack(blocks)), "RS"


# ------------------------------------------- MoE dispatch + grouped GEMM, combine
def _moe_cases(seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i, tile in enumerate(2 * [0, 1, 2, 3, 4, 5, 6, 7, 8, 0, 5, 10]):
        bt = int(rng.choice([64, 128, 256]))
        T = bt * int(rng.integers(1, 5))
        H = int(rng.choice([128, 256, 384] if tile in (5, 6, 7, 8) and rng.random() < 0.8 else [8, 128, 136, 256, 384]))
        E = int(rng.integers(8, 300))
        k = int(rng.integers(1, min(9, E + 1)))
        L = int(rng.integers(1, min(E, 40) + 1))
        eb = int(rng.integers(0, E - L + 1))
        F = 8 * int(rng.integers(1, 70))
        lau = dict(tile=tile, n_copy=int(rng.choice([0, 0, 1, 3])),
                   mode=int(rng.choice([0, 0, 1])), queue_mode=int(rng.choice([0, 1, 2, 3, 4, 5])),
                   grid=int(rng.choice([0, 0, 5, 40])))
        out.append((i, T, H, E, k, L, eb, F, bt, lau))
    return out


@pytest.mark.parametrize("case", _moe_cases(), ids=lambda c: f"moe{c[0]}")
def test_fuzz_moe_dispatch_gemm_and_combine(gpu, case):
    from tile_pipelined_gemm_amd.harness import MoeProblem, bf16_tensor, to_numpy
    i, T, H, E, k, L, eb, F, bt, lau = case
    print(f"MoE case {i}: T={T} H={H} E={E} k={k} L={L} expert_begin={eb} F={F} block_tokens={bt} launch={lau}",
          flush=True)
    w = wl.make_moe(T, H, E, k, L, F, seed=300 + i, dist="int", block_tokens=bt, out_dtype="f32", expert_begin=eb)
    prob = MoeProblem(w)
    prob.Xs.fill_(float("nan"))
    rc = prob.run(launch=gpu.make_launch(**lau), check=False)
    if lau["tile"] in (9, 10, 11) or (lau["tile"] in (5, 6, 7, 8) and H % 128):
        assert rc == gpu.MK_ERR_UNSUPPORTED
        return
    assert rc == gpu.MK_OK, gpu.load().mk_last_error()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, eb, "f32")
    got = prob.outputs()
    for key in ("topk", "counts", "offsets", "perm"):
        assert np.array_equal(got[key], ref[key]), key
    assert got["n_local"] == ref["n_local"]
    assert np.array_equal(got["Y"], ref["Y"])
    # the combine on this dispatch's routing, with seeded expert outputs
    Yl, Yp = wl.moe_combine_inputs(w, seed=400 + i)
    out = torch.full((T, F), float("nan"), dtype=torch.float32, device="cuda")
    ws = gpu.workspace(gpu.mk_moe_combine_workspace(T, k), "cuda")
    gpu.mk_moe_combine(prob.logits, prob.topk, prob.offsets, prob.perm, eb, L, bf16_tensor(Yl), bf16_tensor(Yp),
                       out, ws)
    torch.cuda.synchronize()
    cref, _ = oc.moe_combine(Yl, Yp, w.logits, ref["topk"], ref["perm"], ref["offsets"], eb, L)
    assert_close(out_to_f64(to_numpy(out), "f32"), cref, "f32", f"combine case {i}")


# ------------------------------------------------------------------ MoE gate
def _gate_cases(n=12, seed=2027):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 700)), 8 * int(rng.integers(1, 160)), 8 * int(rng.integers(1, 40)))
            for i in range(n)]


@pytest.mark.parametrize("case", _gate_cases(), ids=lambda c: f"gate{c[0]}")
def test_fuzz_gate(gpu, case):
    from tile_pipelined_gemm_amd.harness import bf16_tensor
    i, T, H, E = case
    print(f"gate case {i}: T={T} H={H} E={E}", flush=True)
    rng = np.random.default_rng(500 + i)
    X = wl.f32_to_bf16_bits(rng.integers(-2, 2, size=(T, H), endpoint=True).astype(np.float32))
    Wg = wl.f32_to_bf16_bits(rng.integers(-2, 2, size=(H, E), endpoint=True).astype(np.float32))
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    ws = gpu.workspace(gpu.mk_moe_gate_workspace(T, H, E))
    gpu.mk_moe_gate(bf16_tensor(X), bf16_tensor(Wg), out, ws)
    torch.cuda.synchronize()
    _, L32 = ogate.gate_logits(X, Wg)
    assert np.array_equal(out.cpu().numpy(), L32)


# ------------------------------------------------------------- ring attention
def _ring_cases(n=12, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.integers(1, 7))
        H = int(rng.integers(1, 5))
        S = int(rng.integers(1, 400))
        lau = dict(grid=int(rng.choice([0, 0, 5, 33])), n_copy=int(rng.choice([0, 0, 1, 4])),
                   mode=int(rng.choice([0, 0, 1])))
        out.append((i, R, H, S, lau))
    return out


@pytest.mark.parametrize("case", _ring_cases(), ids=lambda c: f"ring{c[0]}")
def test_fuzz_ring(gpu, case):
    from tile_pipelined_gemm_amd.harness import RingProblem
    i, R, H, S, lau = case
    print(f"ring case {i}: R={R} H={H} S={S} D=128 launch={lau}", flush=True)
    w = wl.make_ring(H, S, 128, R, seed=600 + i, step_delay_ns=1000, out_dtype="f32")
    prob = RingProblem(w)
    prob.O.fill_(float("nan"))
    if prob.Kr is not None:
        prob.Kr.fill_(float("nan"))
        prob.Vr.fill_(float("nan"))
    prob.run(launch=gpu.make_launch(**lau))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), "f32"), O64, "f32", f"ring case {i}")
