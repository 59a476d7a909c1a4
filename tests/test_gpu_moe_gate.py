"""MoE gate GEMM on the GPU (through the C ABI) against the float64 oracle:
every split of the contraction (8, 4, 2 parts and none, the register-staged
engine for H not a multiple of 128), ragged token counts, integer inputs bit
for bit, repeated calls bit for bit, the full MoE shape on every logit, and the
gate feeding the dispatch + grouped GEMM, whose routing is then bit-exact
against the oracle's routing of the same float32 logits."""
import numpy as np
import pytest
import torch

import oracle.moe as om
import oracle.moe_gate as og
from oracle.numerics import out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _gate(gpu, X, Wg):
    from tile_pipelined_gemm_amd.harness import bf16_tensor
    T, H = X.shape
    E = Wg.shape[1]
    x, w = bf16_tensor(X), bf16_tensor(Wg)
    out = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    ws = gpu.workspace(gpu.mk_moe_gate_workspace(T, H, E))
    gpu.mk_moe_gate(x, w, out, ws)
    torch.cuda.synchronize()
    return out, (x, w, ws)


def _inputs(T, H, E, seed, dist="normal"):
    rng = np.random.default_rng(seed)
    if dist == "int":
        X = wl.f32_to_bf16_bits(rng.integers(-2, 2, size=(T, H), endpoint=True).astype(np.float32))
        W = wl.f32_to_bf16_bits(rng.integers(-2, 2, size=(H, E), endpoint=True).astype(np.float32))
    else:
        X = wl.f32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
        W = wl.f32_to_bf16_bits(rng.standard_normal((H, E), dtype=np.float32) / np.float32(np.sqrt(H)))
    return X, W


@pytest.mark.parametrize("T,H,E", [(200, 1024, 64),     # 2 tiles: the contraction in 8 parts, ragged rows
                                   (1000, 256, 136),    # 16 tiles, 2 parts; E ragged
                                   (4096, 128, 256),    # 64 tiles, one 128-deep unit: no split
                                   (96, 200, 40)])      # H % 128 != 0: register-staged engine, no split
def test_matches_oracle(gpu, T, H, E):
    X, W = _inputs(T, H, E, seed=T + H + E)
    out, _ = _gate(gpu, X, W)
    L64, _ = og.gate_logits(X, W)
    assert_close(out.cpu().numpy().astype(np.float64), L64, "f32", f"gate {T}x{H}x{E}")


@pytest.mark.parametrize("T,H,E", [(200, 1024, 64), (300, 768, 96), (96, 200, 40)])
def test_integer_inputs_bit_exact(gpu, T, H, E):
    # every partial sum is an integer below 2^24: any split and order is exact
    X, W = _inputs(T, H, E, seed=7 + T, dist="int")
    out, _ = _gate(gpu, X, W)
    _, L32 = og.gate_logits(X, W)
    assert np.array_equal(out.cpu().numpy(), L32)


def test_repeated_calls_bit_identical_and_workspace_reusable(gpu):
    X, W = _inputs(512, 2048, 128, seed=11)
    out, (x, w, ws) = _gate(gpu, X, W)
    first = out.clone()
    for _ in range(3):
        out.fill_(float("nan"))
        gpu.mk_moe_gate(x, w, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, first)


def test_full_size_moe_shape_every_logit(gpu):
    w = wl.CONFIGS["moe"]["make"]()
    Wg = wl.moe_gate_weights(w)
    out, _ = _gate(gpu, w.X, Wg)
    L64, _ = og.gate_logits(w.X, Wg)
    assert_close(out.cpu().numpy().astype(np.float64), L64, "f32", "gate 4096x7168x256")


def test_gate_feeds_dispatch_and_grouped_gemm(gpu):
    # gate -> routing -> dispatch -> grouped GEMM, all on the GPU; routing
    # decisions are taken on the same float32 logits on both sides
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.make_moe(1024, 512, 64, 4, 16, 256, seed=81, block_tokens=128)
    Wg = wl.moe_gate_weights(w, seed=81)
    out, _ = _gate(gpu, w.X, Wg)
    L64, _ = og.gate_logits(w.X, Wg)
    logits = out.cpu().numpy()
    assert_close(logits.astype(np.float64), L64, "f32", "gate")
    prob = MoeProblem(w)
    prob.logits.copy_(out)
    prob.Xs.fill_(float("nan"))
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    got = prob.outputs()
    ref = om.moe_dispatch_gemm(w.X, logits, w.W, w.k, w.expert_begin, "bf16")
    for key in ("topk", "counts", "offsets", "perm"):
        assert np.array_equal(got[key], ref[key]), key
    assert_close(out_to_f64(got["Y"], "bf16"), ref["Y64"], "bf16", "gate -> MoE")
