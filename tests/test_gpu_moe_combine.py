"""MoE combine on the GPU (through the C ABI) against the CPU oracle: the
combine alone on seeded expert outputs (the routing and dispatch of both
sides computed independently), ragged widths and the extreme k, and the
chain dispatch + grouped GEMM + combine end to end."""
import numpy as np
import pytest
import torch

import oracle.moe as om
import oracle.moe_combine as oc
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _combine(gpu, prob, Yl, Yp, out_dtype):
    from tile_pipelined_gemm_amd.harness import bf16_tensor, to_numpy
    w = prob.w
    yl = bf16_tensor(Yl)
    yp = bf16_tensor(Yp)
    out = torch.full((w.T, w.F), float("nan"), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                     device="cuda")
    ws = gpu.workspace(gpu.mk_moe_combine_workspace(w.T, w.k), "cuda")
    gpu.mk_moe_combine(prob.logits, prob.topk, prob.offsets, prob.perm, w.expert_begin, w.L, yl, yp, out, ws)
    torch.cuda.synchronize()
    return to_numpy(out)


def _dispatch(gpu, w):
    from tile_pipelined_gemm_amd.harness import MoeProblem
    prob = MoeProblem(w)
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_combine_alone_matches_oracle(gpu, out_dtype):
    w = wl.make_moe(320, 128, 64, 6, 12, 264, seed=51, expert_begin=20, block_tokens=64)
    prob = _dispatch(gpu, w)
    Yl, Yp = wl.moe_combine_inputs(w, seed=2)
    got = _combine(gpu, prob, Yl, Yp, out_dtype)
    topk = om.route_topk(w.logits, w.k)
    _, offsets, perm = om.dispatch(topk, w.E)
    ref, _ = oc.moe_combine(Yl, Yp, w.logits, topk, perm, offsets, w.expert_begin, w.L)
    assert_close(out_to_f64(got, out_dtype), ref, out_dtype, f"combine {out_dtype}")


@pytest.mark.parametrize("k,E,F", [(1, 16, 8), (16, 64, 2056), (8, 256, 2048)])
def test_combine_extreme_k_and_widths(gpu, k, E, F):
    # F = 2056: one 8-column group past the 256 threads' first pass
    w = wl.make_moe(96, 128, E, k, 4, F, seed=52 + k, expert_begin=1, block_tokens=32)
    prob = _dispatch(gpu, w)
    Yl, Yp = wl.moe_combine_inputs(w, seed=3)
    got = _combine(gpu, prob, Yl, Yp, "f32")
    topk = om.route_topk(w.logits, w.k)
    _, offsets, perm = om.dispatch(topk, w.E)
    ref, _ = oc.moe_combine(Yl, Yp, w.logits, topk, perm, offsets, 1, 4)
    assert_close(out_to_f64(got, "f32"), ref, "f32", f"combine k={k} F={F}")


def test_dispatch_gemm_combine_chain(gpu):
    w = wl.make_moe(512, 256, 32, 4, 8, 256, seed=53, expert_begin=8, block_tokens=128)
    prob = _dispatch(gpu, w)
    _, Yp = wl.moe_combine_inputs(w, seed=4)
    from tile_pipelined_gemm_amd.harness import to_numpy
    got = _combine(gpu, prob, to_numpy(prob.Y), Yp, "bf16")
    ref = om.moe_dispatch_gemm(w.X, w.logits, w.W, w.k, 8, "bf16")
    out, _ = oc.moe_combine(ref["Y"], Yp, w.logits, ref["topk"], ref["perm"], ref["offsets"], 8, w.L)
    assert_close(out_to_f64(got, "bf16"), out, "bf16", "dispatch + GEMM + combine")


def test_full_size_combine_config(gpu):
    # the benchmark's combine: T = 4096, H = 7168, top-8 of 256 experts, 32 local
    # experts, F = 2048; every token compared with the oracle's own routing
    w = wl.CONFIGS["moe"]["make"]()
    prob = _dispatch(gpu, w)
    Yl, Yp = wl.moe_combine_inputs(w, seed=0)
    got = _combine(gpu, prob, Yl, Yp, "bf16")
    topk = om.route_topk(w.logits, w.k)
    _, offsets, perm = om.dispatch(topk, w.E)
    ref, _ = oc.moe_combine(Yl, Yp, w.logits, topk, perm, offsets, w.expert_begin, w.L)
    assert_close(out_to_f64(got, "bf16"), ref, "bf16", "combine T=4096 k=8 F=2048")
