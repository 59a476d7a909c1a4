"""The AllGather -> GEMM entry point that allocates nothing
(mk_ag_gemm_noalloc: the library's built-in per-GPU scratch instead of a
workspace), through the C ABI, against mk_ag_gemm on the same inputs: two
calls in a row, the second with a smaller input, each bit-identical to the
entry point with a workspace (same kernels, same arithmetic order)."""
import numpy as np
import pytest
import torch

import oracle.ag_gemm as og
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _both(gpu, w, launch=None):
    from tile_pipelined_gemm_amd.harness import AgProblem, to_numpy
    prob = AgProblem(w)
    prob.C.fill_(float("nan"))
    prob.Ag.fill_(float("nan"))
    prob.run(launch=launch)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    want_C, want_Ag = prob.output().copy(), to_numpy(prob.Ag).copy()
    prob.C.fill_(float("nan"))
    prob.Ag.fill_(float("nan"))
    gpu.mk_ag_gemm_noalloc(prob.shards, prob.B, prob.C, prob.Ag, order=w.order, delay_ns=w.delay_ns,
                           unit_rows=w.unit_rows, launch=launch)
    torch.cuda.synchronize()
    return prob.output(), to_numpy(prob.Ag), want_C, want_Ag


def test_noalloc_two_calls_second_smaller_match_workspace_entry_point(gpu):
    big = wl.make_ag(8, 256, 1024, 768, seed=91, unit_rows=64, max_delay_ns=5000)      # 2048 x 768, 32 units
    small = wl.make_ag(2, 96, 256, 264, seed=92, unit_rows=32, max_delay_ns=2000)     # ragged, 6 units
    for w in (big, small):
        got_C, got_Ag, want_C, want_Ag = _both(gpu, w)
        assert np.array_equal(got_C, want_C)
        assert np.array_equal(got_Ag, want_Ag)
        C64, _ = og.ag_gemm(w.shards, w.B, w.out_dtype)
        assert_close(out_to_f64(got_C, w.out_dtype), C64, w.out_dtype, "noalloc AG")


def test_noalloc_unfused_and_tile_variants(gpu):
    w = wl.make_ag(4, 128, 512, 512, seed=93, dist="int", unit_rows=64, out_dtype="f32")
    _, C = og.ag_gemm(w.shards, w.B, "f32")
    for lau in [gpu.make_launch(mode=1), gpu.make_launch(tile=gpu.TILE_128x128), gpu.make_launch(grid=7)]:
        got_C, _, want_C, _ = _both(gpu, w, launch=lau)
        assert np.array_equal(got_C, want_C)
        assert np.array_equal(got_C, C)
