"""GEMM -> ReduceScatter on the GPU (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle.gemm_rs as orc
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _run(gpu, w, launch=None):
    from tile_pipelined_gemm_amd.harness import RsProblem
    prob = RsProblem(w)
    for o in prob.out:
        o.fill_(float("nan"))
    prob.run(launch=launch)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_small_matches_oracle(gpu, out_dtype):
    # 4 owners of 128 rows, ragged N, several tiles
    w = wl.make_rs(512, 200, 264, 4, seed=21, out_dtype=out_dtype)
    prob = _run(gpu, w)
    S, blocks, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    assert_close(out_to_f64(prob.output(), out_dtype), S, out_dtype, f"RS {out_dtype}")


def test_integer_inputs_bit_exact(gpu):
    w = wl.make_rs(512, 256, 256, 4, seed=22, dist="int")
    prob = _run(gpu, w)
    _, _, outs = orc.gemm_rs(w.A, w.B, w.partials, w.R, "f32")
    assert np.array_equal(prob.output(), np.vstack(outs))


def test_dma_tile_integer_inputs_bit_exact(gpu):
    # K = 256 and 256 rows per owner take the direct-to-LDS 256x256 tile with the
    # reduction done from the accumulators; N = 264 is ragged.
    w = wl.make_rs(1024, 256, 264, 4, seed=26, dist="int")
    prob = _run(gpu, w)
    _, _, outs = orc.gemm_rs(w.A, w.B, w.partials, w.R, "f32")
    assert np.array_equal(prob.output(), np.vstack(outs))


def test_roles_and_baseline_bitwise_identical(gpu):
    w = wl.make_rs(1024, 512, 512, 4, seed=23)
    outs = []
    # the fp32 sum order (local, P_1, ..., P_{R-1}) and the K-loop order do not
    # depend on the role split, the tile shape or fusion, so the bits must agree
    for lau in [dict(), dict(n_reduce=-1), dict(n_reduce=16), dict(n_reduce=64, grid=96), dict(mode=1),
                dict(tile=2), dict(tile=2, n_reduce=32), dict(tile=5, n_reduce=8), dict(tile=5, mode=1),
                dict(tile=3), dict(tile=4), dict(tile=6), dict(tile=7), dict(tile=8)]:
        prob = _run(gpu, w, gpu.make_launch(**lau))
        outs.append(prob.output())
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"variant {i} differs"


def test_xcd_band_queues_same_bits(gpu):
    # queue_mode 1 only changes which workgroup takes which tile: 8 tile
    # columns of 256 (and 16 of 128) split over the 8 per-XCD queues, and the
    # bits equal the one-queue default's for every role split, tile, grid and
    # the unfused baseline; integer inputs are exact against the oracle
    w = wl.make_rs(2048, 256, 2048, 4, seed=27)
    base = _run(gpu, w).output()
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    assert_close(out_to_f64(base, "f32"), S, "f32", "RS one queue")
    for lau in [dict(queue_mode=1), dict(queue_mode=1, tile=2), dict(queue_mode=1, n_reduce=16),
                dict(queue_mode=1, mode=1), dict(queue_mode=1, grid=40), dict(queue_mode=1, grid=3),
                dict(queue_mode=1, tile=5)]:
        got = _run(gpu, w, gpu.make_launch(**lau)).output()
        assert np.array_equal(got, base), f"variant {lau} differs"
    wi = wl.make_rs(2048, 256, 2048, 4, seed=28, dist="int")
    _, _, outs = orc.gemm_rs(wi.A, wi.B, wi.partials, wi.R, "f32")
    assert np.array_equal(_run(gpu, wi, gpu.make_launch(queue_mode=1)).output(), np.vstack(outs))
    # under an arrival schedule the queue rows are the tile rows in landing order
    wa = _arrival_workload("normal", M=1024, N=2048, R=4, unit_rows=128, seed=29)
    ref = _run_arrival(gpu, wa).output()
    for lau in [dict(queue_mode=1), dict(queue_mode=1, n_copy=3), dict(queue_mode=1, mode=1)]:
        got = _run_arrival(gpu, wa, launch=gpu.make_launch(**lau)).output()
        assert np.array_equal(got, ref), f"arrival variant {lau} differs"


@pytest.mark.parametrize("tile", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n_reduce", [8, -1])
def test_every_tile_config(gpu, tile, n_reduce):
    # ragged N; K = 136 (K = 256 for the direct-to-LDS tiles, which need K % 128 == 0)
    w = wl.make_rs(1024, 256 if tile >= 5 else 136, 392, 4, seed=24)
    prob = _run(gpu, w, gpu.make_launch(tile=tile, n_reduce=n_reduce))
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    assert_close(out_to_f64(prob.output(), "f32"), S, "f32", f"RS tile {tile}")


def test_dma_tile_rejects_k_not_multiple_of_128(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = wl.make_rs(1024, 136, 256, 4, seed=27)
    prob = RsProblem(w)
    assert prob.run(launch=gpu.make_launch(tile=5), check=False) == gpu.MK_ERR_UNSUPPORTED


def test_owner_map_in_tile_log(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = wl.make_rs(2048, 64, 512, 8, seed=25)
    prob = RsProblem(w)
    n_tiles = (2048 // 128) * (512 // 128)
    log = torch.full((8 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_128x128, n_reduce=16, tile_log=log))
    torch.cuda.synchronize()
    L = log.cpu().numpy().reshape(-1, 8)
    for t in range(n_tiles):
        tm = t // 4
        assert L[t, 0] == orc.tile_owner(tm, 128, w.M, w.R)
        assert L[t, 3] == -1                                    # no arrival schedule
    assert sorted(L[:, 1].tolist()) == list(range(n_tiles))     # each production slot used once


def test_owner_map_in_tile_log_dma_tile(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = wl.make_rs(2048, 256, 512, 8, seed=28)
    prob = RsProblem(w)
    n_tiles = (2048 // 256) * (512 // 256)
    log = torch.full((8 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(tile=5, tile_log=log))
    torch.cuda.synchronize()
    L = log.cpu().numpy().reshape(-1, 8)
    for t in range(n_tiles):
        assert L[t, 0] == orc.tile_owner(t // 2, 256, w.M, w.R)
        assert L[t, 1] == t


# ---- partial sums under an arrival schedule: units (peer, row block) ----
def _arrival_workload(dist="normal", M=1024, N=264, R=4, unit_rows=128, seed=61):
    # K = 256: the direct-to-LDS 256x256 default tile; N = 264 ragged
    return wl.make_rs(M, 256, N, R, seed=seed, dist=dist, unit_rows=unit_rows, max_delay_ns=20000)


def _run_arrival(gpu, w, landing=True, launch=None, order=None, delay_ns=None):
    from tile_pipelined_gemm_amd.harness import RsProblem
    prob = RsProblem(w, landing=landing)
    for o in prob.out:
        o.fill_(float("nan"))
    if landing:
        for b in prob.landing:
            b.fill_(float("nan"))                  # a tile that read before its unit landed shows NaN
    prob.run(launch=launch, order=order, delay_ns=delay_ns)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


def test_arrival_integer_inputs_bit_exact(gpu):
    w = _arrival_workload("int")
    _, _, outs = orc.gemm_rs(w.A, w.B, w.partials, w.R, "f32", order=w.order, delay_ns=w.delay_ns,
                             unit_rows=w.unit_rows)
    for landing in (True, False):
        prob = _run_arrival(gpu, w, landing=landing)
        assert np.array_equal(prob.output(), np.vstack(outs)), f"landing={landing}"
        if landing:                                # the landing buffers hold the partial sums
            for q in range(w.R - 1):
                assert np.array_equal(prob.landing[q].cpu().numpy(), w.partials[q])


def test_arrival_outputs_independent_of_schedule(gpu):
    # the sum order is fixed, so every schedule, landing choice, role split and
    # the unfused baseline give the bits of the resident path
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = _arrival_workload("normal")
    n = len(w.order)
    base = RsProblem(w)
    for o in base.out:
        o.fill_(float("nan"))
    base.run(arrival=False)                        # every partial sum resident: no schedule
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(base.ws) == gpu.MK_OK
    resident = base.output()
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    assert_close(out_to_f64(resident, "f32"), S, "f32", "RS resident")
    rev = w.order[::-1].copy()
    ident = np.arange(n, dtype=np.int32)
    for kw in [dict(), dict(order=rev), dict(order=ident, delay_ns=np.zeros(n, np.uint32)),
               dict(launch=gpu.make_launch(n_copy=8)), dict(launch=gpu.make_launch(n_copy=1)),
               dict(launch=gpu.make_launch(n_reduce=16)), dict(launch=gpu.make_launch(mode=1)),
               dict(launch=gpu.make_launch(copy_kib=8)), dict(launch=gpu.make_launch(grid=40, n_copy=3)),
               dict(landing=False), dict(landing=False, order=rev), dict(landing=False, launch=gpu.make_launch(mode=1)),
               dict(launch=gpu.make_launch(tile=2)), dict(launch=gpu.make_launch(tile=2, n_reduce=8))]:
        got = _run_arrival(gpu, w, **kw).output()
        assert np.array_equal(got, resident), f"variant {kw} differs"


def test_arrival_units_spanning_tiles_and_all_reduce(gpu):
    # 64-row units under 256-row tiles (four row blocks per tile); the
    # all-reduce of the same contributions equals the owner blocks stacked
    from tile_pipelined_gemm_amd.harness import ArProblem
    w = _arrival_workload("normal", M=1024, N=512, R=4, unit_rows=64, seed=62)
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    rs = _run_arrival(gpu, w).output()
    assert_close(out_to_f64(rs, "f32"), S, "f32", "RS 64-row units")
    ar = ArProblem(w, landing=True)
    ar.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(ar.ws) == gpu.MK_OK
    for o in ar.outputs():
        assert np.array_equal(o, rs)


def test_arrival_tile_and_copy_logs(gpu):
    # every copy item logged once, in arrival order of its units; every tile's
    # reduction became ready only after every copy item of every peer's units
    # under its rows had landed (an item's end stamp is taken once its stores
    # are complete, before its release)
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = _arrival_workload("normal", M=1024, N=512, R=4, unit_rows=128, seed=63)
    prob = RsProblem(w, landing=True)
    n_tiles = (1024 // 256) * (512 // 256)
    parts = 128 * 512 * 4 // (64 * 1024)           # 64 KiB copy items: 4 per unit
    n_units = (w.R - 1) * (w.M // 128)
    tlog = torch.full((8 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    clog = torch.full((8 * n_units * parts,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(tile=gpu.TILE_256x256_DMA, tile_log=tlog, copy_log=clog, copy_kib=64))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    T = tlog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    CL = clog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    assert sorted(map(tuple, CL[:, :2].tolist())) == [(u, p) for u in range(n_units) for p in range(parts)]
    assert [int(CL[i * parts, 0]) for i in range(n_units)] == [int(u) for u in w.order]
    base = int(min(T[:, 4].min(), CL[:, 3].min()))
    rel = lambda x: (int(x) - base) & 0xffffffff
    end_of = {}
    for u, _, _, _, t_end in CL[:, :5]:
        end_of.setdefault(int(u), []).append(rel(t_end))
    for t in range(n_tiles):
        tm = t // 2
        owner, _, wg, b0, t_take, t_ready, t_done, _ = T[t]
        assert owner == orc.tile_owner(tm, 256, w.M, w.R)
        assert b0 == tm * 256 // 128
        assert rel(t_take) <= rel(t_ready) <= rel(t_done)
        units = {orc.unit_of(p, r, w.M, 128) for p in range(1, w.R) for r in (tm * 256, tm * 256 + 255)}
        ends = [e for u in units for e in end_of[u]]
        assert len(ends) == len(units) * parts
        assert rel(t_ready) >= max(ends), f"tile {t} reduced before its partial sums landed"


def test_arrival_withheld_unit_times_out_and_kernel_exits(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = _arrival_workload("normal", seed=64)
    prob = RsProblem(w, landing=True)
    prob.run(withhold=int(w.order[5]), launch=gpu.make_launch(spin_limit_us=20000))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_ERR_TIMEOUT
    # the workspace is reusable and the status was cleared
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    assert_close(out_to_f64(prob.output(), "f32"), S, "f32", "RS after timeout")


def test_full_size_rs_config_whole_output(gpu):
    # every element of the 8 owner blocks against the float64 oracle; the
    # owner blocks stacked are the whole reduced sum (reduce-scatter over all
    # owners equals the all-reduce)
    from tests.full_refs import rs_reduced_sum, rs_workload
    w = rs_workload()
    prob = _run(gpu, w)
    assert_close(out_to_f64(prob.output(), "f32"), rs_reduced_sum(), "f32", "RS 8192x3584x8192")
