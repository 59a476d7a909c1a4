"""The per-shape plan (mk_plan) passed back as the launch gives the same bits
as the default launch of each operation."""
import numpy as np
import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu


def _same(gpu, prob, plan, outputs):
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    want = outputs()
    prob.run(launch=plan)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    got = outputs()
    for a, b in zip(want, got):
        assert np.array_equal(a, b)


def test_plan_ag(gpu):
    from tile_pipelined_gemm_amd.harness import AgProblem
    for w in (wl.make_ag(4, 96, 1024, 640, seed=60, unit_rows=32, max_delay_ns=3000),
              wl.make_ag(8, 16, 1024, 1024, seed=61)):
        prob = AgProblem(w)
        plan = gpu.mk_plan(gpu.MK_OP_AG_GEMM, w.M, w.N, w.K, w.R)
        _same(gpu, prob, plan, lambda: [prob.output().copy()])


def test_plan_rs_and_ar(gpu):
    from tile_pipelined_gemm_amd.harness import RsProblem, ArProblem
    w = wl.make_rs(1024, 512, 768, 4, seed=62, out_dtype="f32")
    prob = RsProblem(w)
    _same(gpu, prob, gpu.mk_plan(gpu.MK_OP_GEMM_RS, w.M, w.N, w.K, w.R),
          lambda: [o.copy() for o in prob.outputs()] if hasattr(prob, "outputs") else [prob.output().copy()])
    prob = ArProblem(w)
    _same(gpu, prob, gpu.mk_plan(gpu.MK_OP_GEMM_AR, w.M, w.N, w.K, w.R),
          lambda: [o.copy() for o in prob.outputs()] if hasattr(prob, "outputs") else [prob.output().copy()])


def test_plan_moe(gpu):
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.make_moe(1024, 256, 64, 8, 16, 512, seed=63, block_tokens=128)
    prob = MoeProblem(w)
    _same(gpu, prob, gpu.mk_plan(gpu.MK_OP_MOE, 0, w.F, w.H), lambda: [prob.outputs()["Y"].copy()])
