"""Ring attention on the GPU (through the C ABI) against the CPU oracle: small
and ragged shapes, one rank, a score range that forces the running max to
move by large steps, receive buffers equal to the ring's shards, outputs
bit-identical across arrival orders, role splits, grids and the unfused
baseline, a withheld unit that times out, and every output of the full-size
configuration."""
import numpy as np
import pytest
import torch

import oracle.ring_attn as ora
from oracle.numerics import bf16_to_f64, f64_to_bf16_bits, out_to_f64
import workloads as wl
from tests.tol import assert_close

pytestmark = pytest.mark.gpu


def _run(gpu, w, **kw):
    from tile_pipelined_gemm_amd.harness import RingProblem
    prob = RingProblem(w)
    prob.O.fill_(float("nan"))
    if prob.Kr is not None:
        prob.Kr.fill_(float("nan"))          # a read before a unit lands would poison the output
        prob.Vr.fill_(float("nan"))
    prob.run(**kw)
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    return prob


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_small_matches_oracle(gpu, out_dtype):
    # 3 query blocks of 128 and 6 key blocks of 64 per shard, 4 ranks
    w = wl.make_ring(2, 384, 128, 4, seed=71, out_dtype=out_dtype)
    prob = _run(gpu, w)
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), out_dtype), O64, out_dtype, f"ring {out_dtype}")


@pytest.mark.parametrize("S,H,R", [(200, 3, 3), (5, 2, 4), (130, 1, 2), (64, 2, 5)])
def test_ragged_sequence_lengths(gpu, S, H, R):
    # S = 200: ragged query block (72 of 128) and key block (8 of 64);
    # S = 5: one partial block; S = 130: two query blocks, the second of 2.
    w = wl.make_ring(H, S, 128, R, seed=72 + S, out_dtype="f32")
    prob = _run(gpu, w)
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), "f32"), O64, "f32", f"ring S={S} H={H} R={R}")


def test_one_rank_is_plain_attention(gpu):
    w = wl.make_ring(2, 256, 128, 1, seed=73)
    prob = _run(gpu, w)
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), "bf16"), O64, "bf16", "ring R=1")


def test_wide_score_range_moves_the_running_max(gpu):
    # Later ring steps carry keys of growing scale, so the row max jumps by
    # more than the rescale threshold at several steps.
    w = wl.make_ring(2, 256, 128, 6, seed=74, out_dtype="f32")
    w.Q = f64_to_bf16_bits(bf16_to_f64(w.Q) * 2.0)
    for s, r in enumerate(ora.ring_order(w.R)):
        w.K[r] = f64_to_bf16_bits(bf16_to_f64(w.K[r]) * (1.0 + 0.75 * s))
    prob = _run(gpu, w)
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), "f32"), O64, "f32", "ring wide scores")


def test_receive_buffers_hold_the_ring_shards(gpu):
    w = wl.make_ring(3, 192, 128, 4, seed=75)
    prob = _run(gpu, w)
    Kr = prob.Kr.view(torch.int16).cpu().numpy().view(np.uint16)
    Vr = prob.Vr.view(torch.int16).cpu().numpy().view(np.uint16)
    for s, r in enumerate(ora.ring_order(w.R)):
        if s == 0:
            continue
        assert np.array_equal(Kr[s - 1], w.K[r]), f"keys of step {s}"
        assert np.array_equal(Vr[s - 1], w.V[r]), f"values of step {s}"


def test_output_independent_of_schedule_roles_and_mode(gpu):
    w = wl.make_ring(4, 320, 128, 4, seed=76)
    base = _run(gpu, w).output()
    rng = np.random.default_rng(5)
    n = (w.R - 1) * w.H
    variants = [
        dict(launch=gpu.make_launch(n_copy=1)),
        dict(launch=gpu.make_launch(n_copy=100000)),
        dict(launch=gpu.make_launch(grid=7)),
        dict(launch=gpu.make_launch(mode=1)),
        dict(order=rng.permutation(n).astype(np.int32), delay_ns=rng.integers(0, 20000, n).astype(np.uint32)),
        dict(order=np.arange(n)[::-1].astype(np.int32), launch=gpu.make_launch(n_copy=2, grid=16)),
    ]
    for kw in variants:
        got = _run(gpu, w, **kw).output()
        assert np.array_equal(got, base), f"variant {kw} differs"


def test_tile_and_copy_logs(gpu):
    w = wl.make_ring(2, 256, 128, 3, seed=77)
    n_items = w.H * 2
    n_copy = 2 * (w.R - 1) * w.H
    tlog = torch.full((8 * n_items,), -1, dtype=torch.int32, device="cuda")
    clog = torch.full((8 * n_copy,), -1, dtype=torch.int32, device="cuda")
    prob = _run(gpu, w, launch=gpu.make_launch(tile_log=tlog, copy_log=clog))
    T = tlog.cpu().numpy().reshape(-1, 8)
    Cl = clog.cpu().numpy().reshape(-1, 8)
    assert sorted(map(tuple, T[:, :2].tolist())) == [(h, b) for h in range(w.H) for b in range(2)]
    assert np.all(T[:, 2] == w.R)
    assert sorted(map(tuple, Cl[:, :2].tolist())) == [(u, p) for u in range((w.R - 1) * w.H) for p in range(2)]
    # copy item w = 2*position + part: the unit in each slot follows the order
    assert np.array_equal(Cl[0::2, 0], w.order) and np.array_equal(Cl[1::2, 0], w.order)
    # consume on arrival: an item's last unit was acquired only after both
    # parts of every unit of its head had landed
    base = int(min(T[:, 5].min(), Cl[:, 3].min()))
    rel = lambda x: (int(x) - base) & 0xffffffff
    for h, _, _, _, _, _, t_ready, _ in T:
        ends = [rel(e) for u, e in zip(Cl[:, 0], Cl[:, 4]) if int(u) % w.H == int(h)]
        assert len(ends) == 2 * (w.R - 1)
        assert rel(t_ready) >= max(ends)


def test_withheld_unit_times_out_and_kernel_exits(gpu):
    from tile_pipelined_gemm_amd.harness import RingProblem
    w = wl.make_ring(2, 256, 128, 3, seed=78)
    prob = RingProblem(w)
    prob.run(withhold=int(w.order[1]), launch=gpu.make_launch(spin_limit_us=20000))
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_ERR_TIMEOUT
    prob.run()
    torch.cuda.synchronize()
    assert gpu.mk_poll_status(prob.ws) == gpu.MK_OK
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), "bf16"), O64, "bf16", "after timeout")


def test_full_size_ring_config_whole_output(gpu):
    # all 16 heads x 4096 queries x 128 dims against the float64 oracle
    w = wl.CONFIGS["ring"]["make"]()
    prob = _run(gpu, w)
    O64, _ = ora.ring_attention(w.Q, w.K, w.V)
    assert_close(out_to_f64(prob.output(), "bf16"), O64, "bf16", "ring 16x4096x128, R = 8")
