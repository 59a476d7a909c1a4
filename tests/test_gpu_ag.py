"""AllGather -> GEMM on the GPU (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle.ag_gemm as og
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _run(gpu, w, **kw):
    from tile_pipelined_gemm_amd.harness import AgProblem
    prob = AgProblem(w)
    prob.Ag.fill_(float("nan"))          # any read before a chunk lands would poison the output
    prob.run(**kw)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


def test_tiny_config_matches_oracle(gpu):
    w = wl.CONFIGS["tiny_ag"]["make"]()
    prob = _run(gpu, w)
    C64, _ = og.ag_gemm(w.shards, w.B, "f32", order=w.order, unit_rows=w.unit_rows)
    assert_close(prob.output().astype(np.float64), C64, "f32", "tiny AG+GEMM")
    # the gathered buffer holds the shards in rank order
    from tile_pipelined_gemm_amd.harness import to_numpy
    assert np.array_equal(to_numpy(prob.Ag), og.gather(w.shards))


def test_integer_inputs_bit_exact(gpu):
    # |partial sums| <= 4K < 2^24: fp32 accumulation is exact, so bits must match.
    w = wl.make_ag(4, 96, 512, 264, seed=5, dist="int", unit_rows=32, out_dtype="f32")
    prob = _run(gpu, w)
    C64, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


@pytest.mark.parametrize("tile", [1, 2, 3, 4])
def test_ragged_shapes_every_tile_config(gpu, tile):
    # M = 300, K = 200, N = 136: ragged in every dimension, several tiles.
    w = wl.make_ag(3, 100, 200, 136, seed=11, unit_rows=20, max_delay_ns=3000)
    prob = _run(gpu, w, launch=gpu.make_launch(tile=tile))
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(prob.output(), "bf16"), C64, "bf16", f"ragged tile {tile}")


def test_mid_size_many_tiles(gpu):
    w = wl.make_ag(8, 128, 1024, 768, seed=12, unit_rows=32, max_delay_ns=20000)
    prob = _run(gpu, w)
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(prob.output(), "bf16"), C64, "bf16", "mid AG")


def test_output_independent_of_schedule_and_roles(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(8, 128, 512, 512, seed=13, unit_rows=32, max_delay_ns=20000)
    prob = AgProblem(w)
    n = w.M // w.unit_rows
    runs = [dict(order=np.arange(n)), dict(order=np.arange(n)[::-1].copy()),
            dict(order=w.order, delay_ns=w.delay_ns),
            dict(order=w.order, launch=gpu.make_launch(n_copy=1)),
            dict(order=w.order, launch=gpu.make_launch(n_copy=64, grid=80)),
            dict(order=w.order, delay_ns=w.delay_ns, launch=gpu.make_launch(copy_kib=16)),
            dict(order=w.order, delay_ns=w.delay_ns, launch=gpu.make_launch(copy_kib=4096, n_copy=3)),
            dict(order=w.order, launch=gpu.make_launch(queue_mode=1)),
            dict(order=w.order, launch=gpu.make_launch(queue_mode=1, grid=80)),
            dict(launch=gpu.make_launch(mode=1)),
            dict(launch=gpu.make_launch(mode=1, queue_mode=1))]
    outs = []
    for kw in runs:
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(**kw)
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
        outs.append(prob.output())
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"run {i} differs"


def test_copy_only_then_gemm_only_equals_fused(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem, to_numpy
    w = wl.make_ag(4, 128, 512, 384, seed=16, unit_rows=64, max_delay_ns=2000)
    prob = AgProblem(w)
    prob.run()
    torch.cuda.synchronize()
    fused = prob.output().copy()
    prob.Ag.fill_(float("nan"))
    prob.C.zero_()
    prob.run(launch=gpu.make_launch(mode=2))           # the baseline's copy kernel alone
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(prob.Ag), og.gather(w.shards))
    prob.run(launch=gpu.make_launch(mode=3))           # its GEMM kernel alone
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    assert np.array_equal(prob.output(), fused)


def test_tile_log_records_chunk_dependencies(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(4, 256, 256, 512, seed=14, unit_rows=64, max_delay_ns=5000)
    prob = AgProblem(w)
    log = torch.full((8 * 64,), -1, dtype=torch.int32, device="cuda")
    clog = torch.full((8 * 64,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(tile=1, tile_log=log, copy_log=clog, copy_kib=16))
    torch.cuda.synchronize()
    L = log.cpu().numpy().reshape(-1, 8).astype(np.int64)
    CL = clog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    n_tiles = (w.M // 256) * (w.N // 256)
    parts = 64 * 256 * 2 // (16 * 1024)              # 16 KiB copy items: 2 per 64-row unit
    n_items = (w.M // 64) * parts
    seen = set()
    for q in range(n_tiles):                      # one record per tile, in queue order
        tm, tn, u0, u1 = L[q, :4]
        assert (u0, u1) == og.tile_units(tm, 256, w.unit_rows, w.M)
        seen.add((tm, tn))
    assert len(seen) == n_tiles
    assert np.all(L[n_tiles:] == -1)
    # copy log: every (unit, part) copied once, in arrival order of units
    items = CL[:n_items]
    assert sorted(map(tuple, items[:, :2].tolist())) == [(u, p) for u in range(w.M // 64) for p in range(parts)]
    assert [int(items[i * parts, 0]) for i in range(w.M // 64)] == [int(c) for c in w.order]
    assert np.all(CL[n_items:] == -1)
    # timestamps (wall clock, 32-bit): a copy item's end stamp is taken once its
    # stores are complete and before its release, so consume-on-arrival means
    # every tile became ready after EVERY copy item of its units had landed;
    # take <= ready <= done; copies start <= end
    wrap = lambda x: x & 0xffffffff
    base = int(min(L[:n_tiles, 5].min(), items[:, 3].min()))
    rel = lambda x: (wrap(x - base))
    for q in range(n_tiles):
        tm, tn, u0, u1, wg, tt, tr, td = L[q]
        assert rel(tt) <= rel(tr) <= rel(td)
        ends = [rel(t_end) for (u, pt, _, _, t_end) in items[:, :5] if u0 <= u <= u1]
        assert len(ends) == (u1 - u0 + 1) * parts
        assert rel(tr) >= max(ends), f"tile {q} ready before its rows landed"
    assert np.all([rel(a) <= rel(b) for a, b in items[:, 3:5]])
    assert gpu.mk_wall_clock_khz() > 0


def test_withheld_chunk_times_out_and_kernel_exits(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(4, 64, 256, 256, seed=15, unit_rows=32)
    prob = AgProblem(w)
    prob.run(withhold=int(w.order[3]), launch=gpu.make_launch(spin_limit_us=20000))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_ERR_TIMEOUT
    # the workspace is reusable and the status was cleared
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(prob.output(), "bf16"), C64, "bf16", "after timeout")


def _whole_output(w, prob, what):
    from tests.full_refs import ag_product
    name = "ag" if w.K == 8192 and w.N == 3584 else "skinny_ag"
    _, C64 = ag_product(name)
    assert_close(out_to_f64(prob.output(), w.out_dtype), C64, w.out_dtype, what)


def test_full_size_ag_config_whole_output(gpu):
    # every one of the 8192 x 3584 outputs against the float64 oracle
    from tests.full_refs import ag_product
    w, _ = ag_product("ag")
    prob = _run(gpu, w)
    from tile_pipelined_gemm_amd.harness import to_numpy
    assert np.array_equal(to_numpy(prob.Ag), og.gather(w.shards))
    _whole_output(w, prob, "AG 8192x8192x3584")


def test_full_size_skinny_config_whole_output(gpu):
    from tests.full_refs import ag_product
    w, _ = ag_product("skinny_ag")
    prob = _run(gpu, w)
    _whole_output(w, prob, "skinny AG 128x8192x28672")


def test_full_size_skinny_config_producer_consumer_tile(gpu):
    # tile 11 at the full skinny shape: the same bits as the 8-slice ring tile
    from tests.full_refs import ag_product
    w, _ = ag_product("skinny_ag")
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_128x128_PC))
    _whole_output(w, prob, "skinny AG 128x8192x28672, producer/consumer tile")
    ref = prob.output().copy()
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128_DMA8))
    torch.cuda.synchronize()
    assert np.array_equal(prob.output(), ref)


# ---- more tiles than workgroups with a partial last round: 272 tiles of
# 256x256 on 256 workgroups ----
def _round_workload(dist, out_dtype):
    # M = 4096, N = 4352: 16 x 17 = 272 tiles; K = 512: 4 K units per tile
    return wl.make_ag(8, 512, 512, 4352, seed=46, dist=dist, unit_rows=128, max_delay_ns=5000,
                      out_dtype=out_dtype)


def test_partial_round_integer_inputs_bit_exact(gpu):
    w = _round_workload("int", "f32")
    prob = _run(gpu, w)
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


def test_partial_round_output_independent_of_grid_mode_and_engine(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = _round_workload("normal", "bf16")
    prob = AgProblem(w)
    outs = []
    for kw in [dict(), dict(grid=80), dict(grid=1), dict(mode=1), dict(queue_mode=1), dict(n_copy=5),
               dict(tile=gpu.TILE_256x256), dict(copy_policy=3), dict(copy_policy=1)]:
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(launch=gpu.make_launch(**kw))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK, kw
        outs.append(prob.output())
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(outs[0], "bf16"), C64, "bf16", "AG, 272 tiles")
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"run {i} differs"


# ---- skinny shapes (M = 128, one tile row; the default tile is the 128x128
# direct-to-LDS tile with the 8-slice ring): every tile shape and engine gives the same bits ----
def test_skinny_integer_inputs_bit_exact(gpu):
    w = wl.make_ag(8, 16, 2048, 8192, seed=47, dist="int", unit_rows=16, max_delay_ns=5000, out_dtype="f32")
    prob = _run(gpu, w)
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


@pytest.mark.parametrize("K", [256, 512])
def test_skinny_default_tile_short_k_ragged(gpu, K):
    # M = 40 (8 shards of 5 rows), N = 392 (ragged): the default skinny tile (the
    # 8-slice ring; K = 256 is exactly one turn of it), integer inputs, exact
    w = wl.make_ag(8, 5, K, 392, seed=58, dist="int", unit_rows=5, max_delay_ns=3000, out_dtype="f32")
    prob = _run(gpu, w)
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128))
    torch.cuda.synchronize()
    assert np.array_equal(prob.output(), C)


def test_skinny_output_independent_of_grid_mode_and_engine(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(8, 16, 2048, 28672, seed=48, unit_rows=16, max_delay_ns=5000)
    prob = AgProblem(w)
    outs = []
    for kw in [dict(), dict(grid=80), dict(grid=3), dict(mode=1), dict(n_copy=5), dict(queue_mode=1),
               dict(tile=gpu.TILE_128x128_DMA), dict(tile=gpu.TILE_128x128), dict(tile=gpu.TILE_128x256),
               dict(tile=gpu.TILE_128x128_DMA8), dict(tile=gpu.TILE_256x128_DMA), dict(tile=gpu.TILE_128x128_PC),
               dict(tile=gpu.TILE_128x128_PC, mode=1), dict(tile=gpu.TILE_128x128_PC, grid=7)]:
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(launch=gpu.make_launch(**kw))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK, kw
        outs.append(prob.output())
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(outs[0], "bf16"), C64, "bf16", "skinny AG")
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"run {i} differs"


# ---- the direct-to-LDS tile engine (tile 5) ----
def test_dma_tile_matches_register_tile_bitwise(gpu):
    # M = 300 and N = 392 are ragged for a 256x256 tile; K = 1024 is a multiple of 128.
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(3, 100, 1024, 392, seed=41, unit_rows=20, max_delay_ns=5000)
    prob = AgProblem(w)
    outs = []
    for tile in (gpu.TILE_256x256, gpu.TILE_256x256_DMA):
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(launch=gpu.make_launch(tile=tile))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
        outs.append(prob.output())
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(outs[1], "bf16"), C64, "bf16", "dma tile")
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("dma,reg", [(6, 2), (7, 3), (8, 4)])
def test_smaller_dma_tiles_match_register_tiles(gpu, dma, reg):
    # 128- and 256-wide direct-to-LDS tiles: ragged M and N, K a multiple of 128
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(3, 100, 384, 392, seed=44, unit_rows=20, max_delay_ns=5000)
    prob = AgProblem(w)
    outs = []
    for tile in (reg, dma):
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(launch=gpu.make_launch(tile=tile))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
        outs.append(prob.output())
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(outs[1], "bf16"), C64, "bf16", f"dma tile {dma}")
    assert np.array_equal(outs[0], outs[1])


def test_deep_ring_dma_tile_matches_register_tile(gpu):
    # the 8-slice ring (tile 9): ragged M and N, K = 768 = three turns of the ring
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(3, 100, 768, 392, seed=49, unit_rows=20, max_delay_ns=5000)
    prob = AgProblem(w)
    outs = []
    for tile in (gpu.TILE_128x128, gpu.TILE_128x128_DMA8, gpu.TILE_128x128_DMA):
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(launch=gpu.make_launch(tile=tile))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
        outs.append(prob.output())
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(outs[1], "bf16"), C64, "bf16", "deep-ring dma tile")
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[2], outs[1])


def test_eight_wave_dma_tile_matches_four_wave_and_register_tiles(gpu):
    # tile 10: 256x256 with 8 waves (two per SIMD); ragged M and N, K = 1024
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(3, 100, 1024, 392, seed=52, unit_rows=20, max_delay_ns=5000)
    prob = AgProblem(w)
    outs = []
    for kw in [dict(tile=gpu.TILE_256x256), dict(tile=gpu.TILE_256x256_DMA_W8),
               dict(tile=gpu.TILE_256x256_DMA), dict(tile=gpu.TILE_256x256_DMA_W8, mode=1),
               dict(tile=gpu.TILE_256x256_DMA_W8, grid=3)]:
        prob.Ag.fill_(float("nan"))
        prob.C.zero_()
        prob.run(launch=gpu.make_launch(**kw))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK, kw
        outs.append(prob.output())
    C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
    assert_close(out_to_f64(outs[1], "bf16"), C64, "bf16", "8-wave dma tile")
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"launch {i} differs"


def test_eight_wave_dma_tile_integer_inputs_bit_exact(gpu):
    w = wl.make_ag(2, 160, 512, 264, seed=53, dist="int", unit_rows=32, out_dtype="f32")
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA_W8))
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


@pytest.mark.parametrize("N,per_row", [(3584, 16), (3000, 16)])
def test_narrow_column_tiles_integer_exact_and_same_bits_as_wide(gpu, N, per_row):
    # The 8-wave 256x256 tile at M = 2048 (8 tile rows) on 64 workgroups:
    # all-256-wide tiles take two rounds (8 x 14 = 112 tiles for N = 3584), so
    # the column plan takes 8 wide and 8 narrow (192-wide) tiles per tile row;
    # for N = 3000 (8 x 12 tiles in two rounds) two rounds of narrow tiles,
    # 16 per tile row, the last 120 columns wide, are shorter still.  The tile
    # log holds one record per tile; the output is exact on integer inputs
    # and the same bits as with 256-wide tiles only (queue_mode 2), the
    # unfused sequence and the GEMM alone.
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(8, 256, 256, N, seed=59, dist="int", unit_rows=128, max_delay_ns=3000, out_dtype="f32")
    prob = AgProblem(w)
    n_tiles = 8 * per_row
    W8 = gpu.TILE_256x256_DMA_W8
    log = torch.full((8 * 8 * 16 * 2,), -1, dtype=torch.int32, device="cuda")   # room for every tile of either plan
    prob.Ag.fill_(float("nan"))
    prob.run(launch=gpu.make_launch(tile=W8, grid=64, tile_log=log))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    L = log.cpu().numpy().reshape(-1, 8)
    assert np.all(L[:n_tiles, 0] >= 0) and np.all(L[n_tiles:] == -1)
    assert sorted(map(tuple, L[:n_tiles, :2].tolist())) == [(tm, tn) for tm in range(8)
                                                             for tn in range(per_row)]
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)
    for kw in [dict(queue_mode=2), dict(mode=1), dict(mode=3), dict(n_copy=1), dict(queue_mode=1)]:
        prob.C.fill_(float("nan"))
        prob.run(launch=gpu.make_launch(tile=W8, grid=64, **kw))
        torch.cuda.synchronize()
        assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK, kw
        assert np.array_equal(prob.output(), C), kw


def test_eight_wave_dma_tile_full_size_ag_config(gpu):
    w = wl.CONFIGS["ag"]["make"]()
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA_W8))
    _whole_output(w, prob, "AG full, 8-wave dma tile")
    ref = prob.output().copy()
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA))
    torch.cuda.synchronize()
    assert np.array_equal(prob.output(), ref)


def test_producer_consumer_tile_matches_register_and_dma_tiles(gpu):
    # tile 11 (one 128-row tile row, A read from its packed copy): M = 120 and
    # N = 392 ragged; K = 640 = 20 slices (one and a quarter turns of the
    # 16-slice ring, so the producers' DMAs past the end are exercised), 128
    # (fewer slices than the ring) and 4096
    from tile_pipelined_gemm_amd.harness import AgProblem
    for K in (640, 128, 4096):
        w = wl.make_ag(3, 40, K, 392, seed=54, unit_rows=20, max_delay_ns=5000)
        prob = AgProblem(w)
        outs = []
        for kw in [dict(tile=gpu.TILE_128x128), dict(tile=gpu.TILE_128x128_PC), dict(tile=gpu.TILE_128x128_DMA),
                   dict(tile=gpu.TILE_128x128_PC, mode=1), dict(tile=gpu.TILE_128x128_PC, grid=3),
                   dict(tile=gpu.TILE_128x128_PC, copy_kib=16), dict(tile=gpu.TILE_128x128_PC, copy_policy=1), dict()]:
            prob.Ag.fill_(float("nan"))
            prob.ws.fill_(255)                     # the packed copy must be rewritten by every call
            prob.ws[:1280].zero_()                 # header and unit counters
            prob.C.zero_()
            prob.run(launch=gpu.make_launch(**kw))
            torch.cuda.synchronize()
            assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK, (K, kw)
            outs.append(prob.output())
        C64, _ = og.ag_gemm(w.shards, w.B, "bf16")
        assert_close(out_to_f64(outs[1], "bf16"), C64, "bf16", f"producer/consumer tile, K={K}")
        for i, o in enumerate(outs[1:], 1):
            assert np.array_equal(outs[0], o), f"K={K} launch {i} differs"


def test_producer_consumer_tile_gemm_alone_packs_the_gathered_rows(gpu):
    # mode 2 gathers (and packs); mode 3 (the GEMM alone) packs a_gathered as
    # it is, so a GEMM after a cleared workspace and a changed a_gathered
    # still follows a_gathered
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(4, 32, 1024, 640, seed=57, unit_rows=32)
    prob = AgProblem(w)
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128_PC, mode=2))
    torch.cuda.synchronize()
    prob.ws.fill_(255)
    prob.ws[:1280].zero_()
    prob.Ag[:32] = -prob.Ag[:32]
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128_PC, mode=3))
    torch.cuda.synchronize()
    got = prob.output().copy()
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128, mode=3))
    torch.cuda.synchronize()
    assert np.array_equal(prob.output(), got)
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK


def test_producer_consumer_tile_integer_inputs_bit_exact(gpu):
    w = wl.make_ag(2, 60, 512, 264, seed=55, dist="int", unit_rows=30, out_dtype="f32")
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_128x128_PC))
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


def test_producer_consumer_tile_rejections(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    lau = gpu.make_launch(tile=gpu.TILE_128x128_PC)
    # K % 128 != 0
    prob = AgProblem(wl.make_ag(2, 64, 320, 128, seed=56))
    assert prob.run(launch=lau, check=False) == gpu.MK_ERR_UNSUPPORTED
    # two tile rows
    prob = AgProblem(wl.make_ag(2, 65, 256, 128, seed=56))
    assert prob.run(launch=lau, check=False) == gpu.MK_ERR_UNSUPPORTED
    # no workspace for the packed copy
    prob = AgProblem(wl.make_ag(2, 64, 256, 128, seed=56))
    rc = gpu.mk_ag_gemm_noalloc(prob.shards, prob.B, prob.C, prob.Ag, launch=lau, check=False)
    assert rc == gpu.MK_ERR_UNSUPPORTED
    # a workspace sized before the packed copy was part of it
    prob.ws = prob.ws[:1280]
    assert prob.run(launch=gpu.make_launch(), check=False) == gpu.MK_ERR_WORKSPACE


def test_deep_ring_dma_tile_integer_inputs_bit_exact(gpu):
    w = wl.make_ag(2, 160, 512, 264, seed=50, dist="int", unit_rows=32, out_dtype="f32")
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_128x128_DMA8))
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


def test_deep_ring_dma_tile_rejects_k_not_multiple_of_256(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(2, 64, 384, 128, seed=51)
    prob = AgProblem(w)
    rc = prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128_DMA8), check=False)
    assert rc == gpu.MK_ERR_UNSUPPORTED


def test_dma_tile_integer_inputs_bit_exact(gpu):
    w = wl.make_ag(2, 160, 512, 264, seed=42, dist="int", unit_rows=32, out_dtype="f32")
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA))
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    assert np.array_equal(prob.output(), C)


def test_dma_tile_rejects_k_not_multiple_of_128(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.make_ag(2, 64, 200, 64, seed=43)
    prob = AgProblem(w)
    rc = prob.run(launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA), check=False)
    assert rc == gpu.MK_ERR_UNSUPPORTED


def test_dma_tile_full_size_ag_config(gpu):
    w = wl.CONFIGS["ag"]["make"]()
    prob = _run(gpu, w, launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA))
    _whole_output(w, prob, "AG full, dma tile")
    ref = prob.output().copy()
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_256x256))
    torch.cuda.synchronize()
    assert np.array_equal(prob.output(), ref)
