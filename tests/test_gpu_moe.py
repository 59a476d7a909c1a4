"""MoE dispatch -> grouped GEMM on the GPU (through the C ABI) against the CPU
oracle: routing, counts, offsets and the dispatch permutation bit-exact, the
grouped GEMM within tolerance."""
import numpy as np
import pytest
import torch

import oracle.moe as om
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _run(gpu, w, **kw):
    from tile_pipelined_gemm_amd.harness import MoeProblem
    prob = MoeProblem(w)
    prob.Xs.fill_(float("nan"))
    prob.run(**kw)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


def _check_exact(prob, ref):
    got = prob.outputs()
    assert np.array_equal(got["topk"], ref["topk"])
    assert np.array_equal(got["counts"], ref["counts"])
    assert np.array_equal(got["offsets"], ref["offsets"])
    assert np.array_equal(got["perm"], ref["perm"])
    assert got["n_local"] == ref["n_local"]
    return got


@pytest.mark.parametrize("eb,L", [(0, 8), (5, 11)])
def test_small_matches_oracle(gpu, eb, L):
    w = wl.make_moe(320, 136, 64, 4, L, 136, seed=31, expert_begin=eb, block_tokens=64)
    prob = _run(gpu, w)
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, eb, "bf16")
    got = _check_exact(prob, ref)
    _check_received(prob, w, ref)
    assert_close(out_to_f64(got["Y"], "bf16"), ref["Y64"], "bf16", "MoE small")


def test_ties_and_signed_zero_routing(gpu):
    rng = np.random.default_rng(32)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0], np.float32)
    logits = vals[rng.integers(0, 5, size=(256, 96))]
    logits[:16] = 0.0
    logits[16:32] = -0.0
    w = wl.make_moe(256, 64, 96, 6, 16, 64, seed=32, logits=logits, block_tokens=32)
    prob = _run(gpu, w, launch=None)
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "bf16")
    _check_exact(prob, ref)
    assert np.all(prob.outputs()["topk"][:32] == np.arange(6))


@pytest.mark.parametrize("E,k", [(300, 8), (1000, 16), (64, 1)])
def test_routing_for_wide_and_narrow_expert_counts(gpu, E, k):
    # E = 300 and 1000 take the 8- and 16-logits-per-lane routing kernels;
    # T = 200 leaves a ragged last routing block of 8 tokens.
    w = wl.make_moe(200, 128, E, k, 6, 128, seed=34 + E, expert_begin=E // 3, block_tokens=40)
    prob = _run(gpu, w)
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, E // 3, "bf16")
    got = _check_exact(prob, ref)
    assert_close(out_to_f64(got["Y"], "bf16"), ref["Y64"], "bf16", f"MoE E={E}")


def test_integer_inputs_bit_exact_f32(gpu):
    w = wl.make_moe(512, 256, 32, 4, 8, 256, seed=33, dist="int", block_tokens=128, out_dtype="f32")
    prob = _run(gpu, w)
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "f32")
    got = _check_exact(prob, ref)
    assert np.array_equal(got["Y"], ref["Y"])


def test_schedule_roles_and_baseline_bitwise_identical(gpu):
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.make_moe(1024, 256, 64, 8, 16, 512, seed=34, block_tokens=128)
    prob = MoeProblem(w)
    nb = len(w.order)
    outs = []
    for kw in [dict(), dict(order=np.arange(nb)[::-1].copy()), dict(delay_ns=np.full(nb, 5000)),
               dict(launch=gpu.make_launch(n_copy=1)), dict(launch=gpu.make_launch(mode=1)),
               dict(launch=gpu.make_launch(tile=2)), dict(launch=gpu.make_launch(tile=gpu.TILE_256x256)),
               dict(launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA)),
               dict(launch=gpu.make_launch(tile=gpu.TILE_128x128_DMA)),
               dict(launch=gpu.make_launch(tile=gpu.TILE_256x128_DMA)),
               dict(launch=gpu.make_launch(tile=gpu.TILE_128x256_DMA)),
               dict(launch=gpu.make_launch(n_copy=3)),
               dict(launch=gpu.make_launch(queue_mode=2)), dict(launch=gpu.make_launch(queue_mode=3)),
               dict(launch=gpu.make_launch(queue_mode=4)), dict(launch=gpu.make_launch(queue_mode=5))]:
        prob.Xs.fill_(float("nan"))
        prob.Y.zero_()
        prob.run(**kw)
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
        o = prob.outputs()
        outs.append(np.concatenate([o["perm"].view(np.uint32), o["Y"].ravel().astype(np.uint32)]))
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"variant {i} differs"


def test_dma_tile_ragged_experts_integer_exact(gpu):
    # H = 384 (a multiple of 128) takes the direct-to-LDS engine; F = 200 is ragged
    # in N and the per-expert row counts are ragged in M.
    w = wl.make_moe(640, 384, 24, 3, 12, 200, seed=36, dist="int", block_tokens=64, out_dtype="f32",
                    expert_begin=6)
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA))
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 6, "f32")
    got = _check_exact(prob, ref)
    assert np.array_equal(got["Y"], ref["Y"])


def test_half_height_tail_tiles_integer_exact(gpu):
    # expert row counts with tails of at most 128 rows (run by the 128x256
    # engine) and of more (the 256x256 one), F ragged: exact on integer inputs,
    # and the same bits as the register-staged engine, which has no half tile
    w = wl.make_moe(2048, 256, 16, 4, 8, 520, seed=39, dist="int", block_tokens=256, out_dtype="f32")
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA))
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "f32")
    tails = [int(c) % 256 for c in ref["counts"][:8]]
    assert any(0 < t <= 128 for t in tails) and any(t > 128 for t in tails), tails
    got = _check_exact(prob, ref)
    assert np.array_equal(got["Y"], ref["Y"])
    y_dma = prob.outputs()["Y"].copy()
    prob.Y.zero_()
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_256x256))
    torch.cuda.synchronize()
    assert np.array_equal(prob.outputs()["Y"], y_dma)


def test_dma_tile_rejects_h_not_multiple_of_128(gpu):
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.make_moe(128, 136, 16, 2, 8, 64, seed=37, block_tokens=64)
    prob = MoeProblem(w)
    assert prob.run(launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA), check=False) == gpu.MK_ERR_UNSUPPORTED


@pytest.mark.parametrize("tile,bm,bn", [(0, 128, 128), (5, 256, 256)])
def test_tile_and_copy_logs(gpu, tile, bm, bn):
    # Every grouped-GEMM tile is logged once with its expert, first row and row
    # count; in the fused mode each tile saw all of its rows landed.  Every
    # (block, part) copy item is logged once and the items copy every local row.
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.make_moe(640, 384, 24, 3, 12, 200, seed=38, block_tokens=64, expert_begin=6)
    prob = MoeProblem(w)
    tiles_n = -(-w.F // bn)
    n_tiles = (w.T * min(w.k, w.L) // 128 + w.L + 1) * tiles_n
    tlog = torch.full((8 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    clog = torch.full((8 * 2 * w.T,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(tile=tile, tile_log=tlog, copy_log=clog))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    counts = prob.outputs()["counts"][6:18]
    want = [(l, r0, min(bm, int(c) - r0)) for l, c in enumerate(counts) for r0 in range(0, int(c), bm)
            for _ in range(tiles_n)]
    T = tlog.cpu().numpy().reshape(-1, 8)
    T = T[T[:, 0] >= 0]
    assert [tuple(int(x) for x in r[:3]) for r in T] == want
    assert np.array_equal(T[:, 3], T[:, 2])
    C = clog.cpu().numpy().reshape(-1, 8)
    C = C[C[:, 0] >= 0]
    parts = 64 // 4                                # copy items of 4 tokens
    assert sorted((int(b), int(q)) for b, q in C[:, :2]) == [(b, q) for b in range(w.T // 64) for q in range(parts)]
    assert int(C[:, 5].sum()) == prob.local_rows()
    # consume on arrival: a tile became ready only after every copy item that
    # holds one of its rows had landed (an item's end stamp is taken once its
    # stores are complete, before it is counted)
    out = prob.outputs()
    perm, offsets = out["perm"], out["offsets"]
    end_of = {(int(b), int(q)): int(e) for b, q, e in zip(C[:, 0], C[:, 1], C[:, 4])}
    base = int(min(T[:, 5].min(), C[:, 3].min()))
    rel = lambda x: (int(x) - base) & 0xffffffff
    for l, r0, n, _, _, _, t_ready, _ in T:
        pos0 = int(offsets[6 + l]) + int(r0)
        toks = perm[pos0:pos0 + int(n)] // w.k
        items = {(int(t) // 64, (int(t) % 64) // 4) for t in toks}
        assert rel(t_ready) >= max(rel(end_of[i]) for i in items)


def _split_tail_workload(dist, out_dtype):
    # 38 M-tiles x 8 N-tiles of 256x256 = 304 tiles: on 256 workgroups a last
    # round of 48 tiles, which is split into 4 K parts of 256
    return wl.make_moe(2048, 1024, 16, 4, 16, 2048, seed=71, block_tokens=256, dist=dist, out_dtype=out_dtype)


def _in_split_regime(w):
    topk = om.route_topk(w.logits, w.k)
    counts, _, _ = om.dispatch(topk, w.E)
    tiles = sum((int(c) + 255) // 256 for c in counts[:w.L]) * (w.F // 256)
    full = torch.cuda.get_device_properties(0).multi_processor_count
    return tiles > full and 0 < tiles % full <= full // 4


def test_split_tail_integer_inputs_bit_exact(gpu):
    w = _split_tail_workload("int", "f32")
    assert _in_split_regime(w), "shape no longer exercises the split tail on this device"
    prob = _run(gpu, w)
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "f32")
    got = _check_exact(prob, ref)
    assert np.array_equal(got["Y"], ref["Y"])


def test_split_tail_bitwise_identical_across_launches(gpu):
    w = _split_tail_workload("normal", "bf16")
    outs = []
    # queue_mode=1: per-XCD queues keyed by tile column (8 column tiles here)
    for kw in [dict(), dict(mode=1), dict(grid=80), dict(n_copy=5), dict(n_copy=64),
               dict(queue_mode=1), dict(queue_mode=1, n_copy=64), dict(queue_mode=1, grid=80),
               dict(queue_mode=1, mode=1),
               dict(queue_mode=3), dict(queue_mode=2), dict(queue_mode=4)]:
        prob = _run(gpu, w, launch=gpu.make_launch(**kw))
        outs.append(prob.outputs()["Y"])
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "bf16")
    assert_close(out_to_f64(outs[0], "bf16"), ref["Y64"], "bf16", "MoE split tail")
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"launch {i} differs"


def test_xcd_queues_with_two_columns_per_queue(gpu):
    # 128x128 tiles: 16 column tiles, two per XCD queue; another tile count, so
    # another split tail than the 256x256 default: compared with its own
    # single-queue launch and with the oracle
    w = _split_tail_workload("normal", "bf16")
    outs = []
    for kw in [dict(tile=gpu.TILE_128x128_DMA), dict(tile=gpu.TILE_128x128_DMA, queue_mode=1),
               dict(tile=gpu.TILE_128x128_DMA, queue_mode=1, n_copy=64)]:
        prob = _run(gpu, w, launch=gpu.make_launch(**kw))
        outs.append(prob.outputs()["Y"])
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "bf16")
    assert_close(out_to_f64(outs[1], "bf16"), ref["Y64"], "bf16", "MoE 128x128 per-XCD queues")
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"launch {i} differs"


def test_withheld_block_times_out(gpu):
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.make_moe(512, 64, 32, 4, 8, 64, seed=35, block_tokens=64)
    prob = MoeProblem(w)
    prob.run(withhold=int(w.order[0]), launch=gpu.make_launch(spin_limit_us=20000))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_ERR_TIMEOUT
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK


def _check_received(prob, w, ref):
    # the receive buffer holds every token with a local expert in its own row;
    # the rows of the other tokens are never written (still the NaN poison)
    from tile_pipelined_gemm_amd.harness import to_numpy
    toks = np.unique(om.landing_tokens(ref["perm"], ref["offsets"], w.k, w.expert_begin, w.L))
    xs = to_numpy(prob.Xs)
    assert np.array_equal(xs[toks], w.X[toks])
    rest = np.setdiff1d(np.arange(w.T), toks)
    assert np.all(np.isnan(prob.Xs[torch.as_tensor(rest, device=prob.Xs.device)].float().cpu().numpy()))


def test_full_size_moe_config_whole_output(gpu):
    # routing, counts, offsets, perm bit-exact; every received token row and
    # every output row (every expert's ragged last M-tile included) against
    # the float64 oracle
    w = wl.CONFIGS["moe"]["make"]()
    prob = _run(gpu, w)
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 0, "bf16")
    got = _check_exact(prob, ref)
    n = ref["n_local"]
    _check_received(prob, w, ref)
    assert_close(out_to_f64(got["Y"][:n], "bf16"), ref["Y64"], "bf16", "MoE full")
