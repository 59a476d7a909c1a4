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
    log = torch.full((2 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(n_reduce=16, tile_log=log))
    torch.cuda.synchronize()
    L = log.cpu().numpy().reshape(-1, 2)
    for t in range(n_tiles):
        tm = t // 4
        assert L[t, 0] == orc.tile_owner(tm, 128, w.M, w.R)
    assert sorted(L[:, 1].tolist()) == list(range(n_tiles))     # each production slot used once


def test_owner_map_in_tile_log_dma_tile(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = wl.make_rs(2048, 256, 512, 8, seed=28)
    prob = RsProblem(w)
    n_tiles = (2048 // 256) * (512 // 256)
    log = torch.full((2 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=gpu.make_launch(tile=5, tile_log=log))
    torch.cuda.synchronize()
    L = log.cpu().numpy().reshape(-1, 2)
    for t in range(n_tiles):
        assert L[t, 0] == orc.tile_owner(t // 2, 256, w.M, w.R)
        assert L[t, 1] == t


def test_full_size_rs_config_sampled(gpu):
    w = wl.CONFIGS["rs"]["make"]()
    prob = _run(gpu, w)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(w.M, 64, replace=False), [0, 1023, 1024, w.M - 1]]))
    ref = orc.gemm_rs_rows(w.A, w.B, w.partials, rows)
    got = out_to_f64(prob.output()[rows], "f32")
    assert_close(got, ref, "f32", "RS 8192x3584x8192")
    # the reduce-scatter over all owners is the all-reduce: every owner block filled
    assert not np.any(np.isnan(prob.output()))
