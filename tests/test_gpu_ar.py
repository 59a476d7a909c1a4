"""GEMM -> AllReduce on the GPU (through the C ABI) against the CPU oracle:
every rank's output holds the whole reduced sum, bit-identical across ranks,
role splits, tile shapes and the unfused baseline, and equal to the
reduce-scatter's owner blocks stacked (same fp32 sum order)."""
import numpy as np
import pytest
import torch

import oracle.gemm_ar as oar
import oracle.gemm_rs as orc
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _run(gpu, w, launch=None):
    from tile_pipelined_gemm_amd.harness import ArProblem
    prob = ArProblem(w)
    for o in prob.out:
        o.fill_(float("nan"))
    prob.run(launch=launch)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


def _same_on_every_rank(outs):
    for r, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"rank {r} differs from rank 0"


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_ragged_shape_matches_oracle(gpu, out_dtype):
    # M = 300 is ragged for every tile height and not a multiple of R = 4
    # (allowed for the all-reduce); N = 264 is ragged too.
    w = wl.make_rs(300, 256, 264, 4, seed=61, out_dtype=out_dtype)
    prob = _run(gpu, w)
    outs = prob.outputs()
    _same_on_every_rank(outs)
    S, _ = oar.gemm_ar(w.A, w.B, w.partials, w.R, out_dtype)
    assert_close(out_to_f64(outs[0], out_dtype), S, out_dtype, f"AR {out_dtype}")


def test_integer_inputs_bit_exact(gpu):
    w = wl.make_rs(512, 256, 264, 8, seed=62, dist="int")
    prob = _run(gpu, w)
    _, ref = oar.gemm_ar(w.A, w.B, w.partials, w.R, "f32")
    for o, r in zip(prob.outputs(), ref):
        assert np.array_equal(o, r)


def test_all_reduce_equals_reduce_scatter_stacked(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = wl.make_rs(1024, 512, 512, 4, seed=63)
    ar = _run(gpu, w).outputs()
    rs = RsProblem(w)
    rs.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(rs.ws) == gpu.MK_OK
    stacked = rs.output()
    for o in ar:
        assert np.array_equal(o, stacked)


def test_roles_tiles_and_baseline_bitwise_identical(gpu):
    w = wl.make_rs(1024, 512, 512, 4, seed=64, out_dtype="bf16")
    outs = []
    for lau in [dict(), dict(n_reduce=-1), dict(n_reduce=16), dict(n_reduce=64, grid=96), dict(mode=1),
                dict(tile=2), dict(tile=2, n_reduce=32), dict(tile=5, mode=1), dict(tile=6), dict(tile=7),
                dict(tile=8), dict(queue_mode=1, tile=2), dict(queue_mode=1, tile=2, n_reduce=16)]:
        o = _run(gpu, w, gpu.make_launch(**lau)).outputs()
        _same_on_every_rank(o)
        outs.append(o[0])
    for i, o in enumerate(outs[1:], 1):
        assert np.array_equal(outs[0], o), f"variant {i} differs"


def test_full_size_config_whole_output(gpu):
    from tests.full_refs import rs_reduced_sum, rs_workload
    w = rs_workload()
    from tile_pipelined_gemm_amd.harness import ArProblem
    prob = ArProblem(w)
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    for r in range(1, w.R):                        # compared on the device: 8 x 256 MiB
        assert torch.equal(prob.out[0], prob.out[r]), f"rank {r} differs"
    assert_close(out_to_f64(prob.out[3].cpu().numpy(), "f32"), rs_reduced_sum(), "f32", "AR 8192x3584x8192")
