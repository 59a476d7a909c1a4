"""Benchmark of the fused tile-pipelined GEMM kernels on one MI355X.

One step = one fused AllGather -> GEMM call at its single-GPU share
(R = 8 shards of 1024 x 8192 bf16, B 8192 x 3584, 128-row chunks arriving in a
seeded order with 0-20 us release delays, bf16 output): the workload the
headline metric is quoted on.  Prints ONE JSON line.  The same line carries
the other single-GPU workloads (GEMM+ReduceScatter, MoE dispatch+grouped
GEMM, the skinny AllGather+GEMM) under "configs", each with its unfused
baseline, plus the roofline of the fused kernel and the CPU-oracle baseline.

Inputs are seeded synthetic tensors (workloads/), resident in HBM before the
timed region.  Several copies of each workload are rotated so consecutive
steps do not find their operands in the 256 MiB last-level (MALL) cache.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6        # 256 CU x 2.4 GHz x 4096 bf16 FLOP/clk/CU (dense)
PEAK_HBM_GBS = 8000.0            # HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


AG_KERNEL_SOURCES = ["mk_ag_gemm.hip", "mk_device.h", "mk_gemm_dma.h", "mk_host.h", "mk_host.hip", "mk_tiles.h"]
AG_COUNTERS = os.path.join(ROOT, "profiles", "ag_gemm_8192x8192x3584_counters.md")
_COMMON = ["mk_device.h", "mk_gemm_dma.h", "mk_host.h", "mk_host.hip", "mk_tiles.h"]
# per workload: (bound, kernel sources whose hash the counter summary records, summary)
ROOFLINES = {
    "ag": ("mfma", AG_KERNEL_SOURCES, AG_COUNTERS),
    "skinny_ag": ("hbm", AG_KERNEL_SOURCES, os.path.join(ROOT, "profiles", "skinny_ag_128x8192x28672.md")),
    "rs": ("hbm", ["mk_gemm_rs.hip"] + _COMMON, os.path.join(ROOT, "profiles", "gemm_rs_8192x3584x8192_r8.md")),
    "ar": ("hbm", ["mk_gemm_rs.hip"] + _COMMON, os.path.join(ROOT, "profiles", "gemm_ar_8192x3584x8192_r8.md")),
    "moe": ("mfma", ["mk_moe.hip"] + _COMMON,
            os.path.join(ROOT, "profiles", "moe_dispatch_gemm_t4096_h7168_e256_k8_f2048.md")),
    "ring": ("mfma", ["mk_ring_attn.hip"] + _COMMON, os.path.join(ROOT, "profiles", "ring_attn_16x4096x128_r8.md")),
}


def counter_traffic(sources, summary, csrc=os.path.join(ROOT, "tile_pipelined_gemm_amd", "csrc")):
    """HBM bytes per launch from a committed rocprofv3 counter summary:
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) times the factors a plain copy
    of known size gave.  None unless the kernel sources still hash to the
    value the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    try:
        with open(summary) as fh:
            kv = dict(ln.split(":", 1) for ln in fh.read().splitlines()
                      if ":" in ln and ln.split(":", 1)[0] in
                      ("source-sha256", "fetch-scale", "write-scale", "FETCH_SIZE_KiB", "WRITE_SIZE_KiB"))
    except OSError:
        return None
    if len(kv) != 5 or kv["source-sha256"].strip() != h.hexdigest():
        return None
    return int(1024 * (float(kv["FETCH_SIZE_KiB"]) * float(kv["fetch-scale"]) +
                       float(kv["WRITE_SIZE_KiB"]) * float(kv["write-scale"])))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", default="", help="comma list of workloads to run (ag,skinny_ag,rs,ar,moe)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the unfused and library yardsticks")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured MFMA and HBM peaks")
    ap.add_argument("--copies", type=int, default=0, help="rotated input copies (0 = auto)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--ag-launch", default="",
                    help="launch options for the primary AG timing, e.g. mode=1,tile=5,n_copy=64,copy_kib=256")
    ap.add_argument("--moe-timeline", default="",
                    help="only run the MoE workload once per launch spec (';'-separated) with the "
                         "tile and copy logs and print each timeline summary as JSON")
    ap.add_argument("--ag-timeline", default="",
                    help="only run the AG workload once per launch spec (';'-separated) with the "
                         "tile and copy logs and print each timeline summary as JSON")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    return ap.parse_args()


class Timing(tuple):
    """(wall ms/step, mean event ms/launch) with the median and minimum of the
    per-launch event times as attributes."""
    median = 0.0
    min = 0.0


def settle(fn, seconds=0.5):
    """Bring the device out of its idle clocks before anything is timed: run fn
    back to back for about `seconds` (the first ~0.5 s of activity runs
    measurably slower).  Part of set-up, like allocating the inputs; the
    warm-up and timed steps come after it."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def timed(fn, steps, warmup, stream):
    """Run fn warmup+steps times; return Timing(wall ms/step, mean event ms/launch)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = sorted(a.elapsed_time(b) for a, b in ev)
    t = Timing((wall, sum(per) / steps))
    t.median = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    t.min = per[0]
    return t


def bench_ag(name, args, stream, extra=True):
    import torch
    import workloads as wl
    from tile_pipelined_gemm_amd import mk
    from tile_pipelined_gemm_amd.harness import AgProblem
    w = wl.CONFIGS[name]["make"](args.seed)
    foot = (sum(s.nbytes for s in w.shards) * 2 + w.B.nbytes + w.M * w.N * 2)
    copies = args.copies or max(1, min(4, int(3 * 256e6 // foot) + 1))
    probs = [AgProblem(w) for _ in range(copies)]
    flops = probs[0].flops
    # algorithmic bytes: gather (read+write A), GEMM reads A and B once, writes C once
    abytes = 2 * w.M * w.K * 2 + w.M * w.K * 2 + w.K * w.N * 2 + w.M * w.N * (2 if w.out_dtype == "bf16" else 4)

    opts = dict(kv.split("=") for kv in args.ag_launch.split(",") if kv) if name == "ag" else {}
    lau0 = mk.make_launch(**{k: int(v) for k, v in opts.items()})

    def fused(i):
        probs[i % copies].run(launch=lau0, stream=stream, check=False)

    if int(opts.get("mode", 0)) == 3:   # the GEMM alone reads a gathered A: gather it once first
        for p in probs:
            p.run(stream=stream, check=False)
    settle(fused)
    tm = timed(fused, args.steps, args.warmup, stream)
    wall, kern = tm
    for p in probs:
        assert mk.mk_poll_status(p.ws, stream) == mk.MK_OK
    r = dict(workload=wl.CONFIGS[name]["desc"], M=w.M, K=w.K, N=w.N, R=w.R, chunk_rows=w.unit_rows,
             copies=copies, ms=wall, kernel_ms=kern, kernel_ms_median=tm.median, kernel_ms_min=tm.min,
             tflops=flops / kern / 1e9, gbs=abytes / kern / 1e6, flops=flops, alg_bytes=abytes)
    if extra:
        lau = mk.make_launch(mode=1)

        def unfused(i):
            probs[i % copies].run(launch=lau, stream=stream, check=False)

        uw, uk = timed(unfused, max(3, args.steps // 2), 2, stream)
        r["unfused_ms"] = uk
        r["speedup_vs_unfused"] = uk / kern
        # role split and scheduling variants of the fused kernel
        variants = [("n_copy64", dict(n_copy=64)), ("copy_writeback", dict(copy_policy=1)),
                    ("copy_kib256", dict(copy_kib=256)),
                    ("xcd_queues", dict(queue_mode=1)),
                    ("copy_only", dict(mode=2)), ("gemm_only", dict(mode=3)),
                    ("gemm_only_xcd_queues", dict(mode=3, queue_mode=1))]
        if w.M >= 256:
            variants += [("tile_reg", dict(tile=mk.TILE_256x256)),
                         ("wide_tiles_only", dict(queue_mode=2)),
                         ("gemm_only_wide_tiles_only", dict(mode=3, queue_mode=2)),
                         ("tile_dma4", dict(tile=mk.TILE_256x256_DMA)),
                         ("gemm_only_dma4", dict(mode=3, tile=mk.TILE_256x256_DMA)),
                         ("copy_kib1024", dict(copy_kib=1024))]
        else:                                        # skinny: the 128-row tiles
            variants += [("tile_128x128", dict(tile=mk.TILE_128x128)),
                         ("tile_128x256_dma", dict(tile=mk.TILE_128x256_DMA)),
                         ("tile_256x128_dma", dict(tile=mk.TILE_256x128_DMA)),
                         ("gemm_only_128x256_dma", dict(mode=3, tile=mk.TILE_128x256_DMA))]
        for tag, kw in variants:
            lv = mk.make_launch(**kw)
            _, vk = timed(lambda i: probs[i % copies].run(launch=lv, stream=stream, check=False), 10, 3, stream)
            r[f"variant_{tag}_ms"] = vk
        # overlap efficiency: the share of the shorter phase hidden by fusion;
        # and against the unfused sequence itself: the share of the copy
        # phase's time that fusion saves (negative when fused is slower)
        tc, tg = r["variant_copy_only_ms"], r["variant_gemm_only_ms"]
        r["overlap_eff"] = (tc + tg - kern) / min(tc, tg)
        r["overlap_eff_vs_unfused"] = (uk - kern) / tc
        # hipBLASLt yardstick on the already gathered A (not the target)
        Ag = [p.Ag for p in probs]
        Bs = [p.B for p in probs]

        def lib(i):
            torch.matmul(Ag[i % copies], Bs[i % copies])

        _, lk = timed(lib, max(3, args.steps // 2), 2, stream)
        r["torch_matmul_ms"] = lk
        r["torch_matmul_tflops"] = flops / lk / 1e9
    return r


def bench_rs(args, stream, extra=True):
    import workloads as wl
    from tile_pipelined_gemm_amd import mk
    from tile_pipelined_gemm_amd.harness import RsProblem
    w = wl.CONFIGS["rs"]["make"](args.seed)
    copies = args.copies or 1      # 2.3 GB of operands per copy: far beyond the MALL already
    probs = [RsProblem(w) for _ in range(copies)]
    del w.partials[:]
    flops = probs[0].flops
    M, K, N, R = probs[0].w.M, probs[0].w.K, probs[0].w.N, probs[0].w.R
    abytes = M * K * 2 + K * N * 2 + (R - 1) * M * N * 4 + M * N * 4

    def fused(i):
        probs[i % copies].run(stream=stream, check=False)

    settle(fused, 0.3)
    wall, kern = timed(fused, max(3, args.steps // 2), 2, stream)
    for p in probs:
        assert mk.mk_poll_status(p.ws, stream) == mk.MK_OK
    r = dict(workload=wl.CONFIGS["rs"]["desc"], M=M, K=K, N=N, R=R, ms=wall, kernel_ms=kern,
             tflops=flops / kern / 1e9, gbs=abytes / kern / 1e6, flops=flops, alg_bytes=abytes,
             hbm_frac=abytes / kern / 1e6 / PEAK_HBM_GBS)
    if extra:
        for nr in (16, 32):
            lau = mk.make_launch(n_reduce=nr)
            _, k2 = timed(lambda i: probs[i % copies].run(launch=lau, stream=stream, check=False), 3, 1, stream)
            r[f"roles_n_reduce{nr}_ms"] = k2
        lau = mk.make_launch(mode=1)
        _, uk = timed(lambda i: probs[i % copies].run(launch=lau, stream=stream, check=False), 3, 1, stream)
        r["unfused_ms"] = uk
        r["speedup_vs_unfused"] = uk / kern
        # the baseline's phases alone: its GEMM kernel (to fp32 staging) and its reduce kernel
        for tag, md in (("gemm_only", 3), ("reduce_only", 2)):
            lv = mk.make_launch(mode=md)
            _, vk = timed(lambda i: probs[i % copies].run(launch=lv, stream=stream, check=False), 3, 1, stream)
            r[f"variant_{tag}_ms"] = vk
        tg, tr = r["variant_gemm_only_ms"], r["variant_reduce_only_ms"]
        r["overlap_eff"] = (tg + tr - kern) / min(tg, tr)
        r["overlap_eff_vs_unfused"] = (uk - kern) / min(tg, tr)
    return r


def bench_ar(args, stream, extra=True):
    """GEMM -> AllReduce on the GEMM+RS inputs: every one of the R ranks'
    outputs receives the whole reduced sum."""
    import workloads as wl
    from tile_pipelined_gemm_amd import mk
    from tile_pipelined_gemm_amd.harness import ArProblem
    w = wl.CONFIGS["rs"]["make"](args.seed)
    prob = ArProblem(w)
    del w.partials[:]
    flops = prob.flops
    M, K, N, R = w.M, w.K, w.N, w.R
    abytes = M * K * 2 + K * N * 2 + (R - 1) * M * N * 4 + R * M * N * 4

    def fused(i):
        prob.run(stream=stream, check=False)

    settle(fused, 0.3)
    wall, kern = timed(fused, max(3, args.steps // 2), 2, stream)
    assert mk.mk_poll_status(prob.ws, stream) == mk.MK_OK
    r = dict(workload="GEMM+AR 8192x3584x8192, 7 fp32 partials, 8 ranks each receive the fp32 sum",
             M=M, K=K, N=N, R=R, ms=wall, kernel_ms=kern, tflops=flops / kern / 1e9, gbs=abytes / kern / 1e6,
             flops=flops, alg_bytes=abytes, hbm_frac=abytes / kern / 1e6 / PEAK_HBM_GBS)
    if extra:
        lau = mk.make_launch(mode=1)
        _, uk = timed(lambda i: prob.run(launch=lau, stream=stream, check=False), 3, 1, stream)
        r["unfused_ms"] = uk
        r["speedup_vs_unfused"] = uk / kern
    return r


def bench_moe(args, stream, extra=True):
    import numpy as np
    import workloads as wl
    from tile_pipelined_gemm_amd import mk
    from tile_pipelined_gemm_amd.harness import MoeProblem
    w = wl.CONFIGS["moe"]["make"](args.seed)
    probs = [MoeProblem(w) for _ in range(args.copies or 2)]
    copies = len(probs)
    probs[0].run(stream=stream)
    stream.synchronize()
    rows = probs[0].local_rows()
    flops = 2.0 * rows * w.H * w.F
    # weights, the received token rows (read from X, written to Xs, read by the
    # tiles), Y and the logits
    recv = probs[0].received_rows()
    abytes = (w.L * w.H * w.F * 2 + 3 * recv * w.H * 2 + rows * w.F * 2 + w.T * w.E * 4)

    def fused(i):
        probs[i % copies].run(stream=stream, check=False)

    settle(fused, 0.3)
    wall, kern = timed(fused, max(3, args.steps // 2), 2, stream)
    for p in probs:
        assert mk.mk_poll_status(p.ws, stream) == mk.MK_OK
    r = dict(workload=wl.CONFIGS["moe"]["desc"], T=w.T, H=w.H, E=w.E, k=w.k, L=w.L, F=w.F, local_rows=rows,
             received_rows=recv,
             ms=wall, kernel_ms=kern, tflops=flops / kern / 1e9, gbs=abytes / kern / 1e6,
             flops=flops, alg_bytes=abytes)
    if extra:
        lau = mk.make_launch(mode=1)
        _, uk = timed(lambda i: probs[i % copies].run(launch=lau, stream=stream, check=False), 5, 2, stream)
        r["unfused_ms"] = uk
        r["speedup_vs_unfused"] = uk / kern
        # the combine step after the grouped GEMM: this rank's tokens gather
        # their k expert rows (local ones from Y, the rest from the peers'
        # returned outputs) weighted by the top-k softmax
        import torch
        Yp = torch.from_numpy(wl.moe_combine_inputs(w, seed=args.seed)[1].view(np.int16)).cuda().view(torch.bfloat16)
        cout = torch.empty(w.T, w.F, dtype=torch.bfloat16, device="cuda")
        cws = mk.workspace(mk.mk_moe_combine_workspace(w.T, w.k))
        p0 = probs[0]

        def combine(i):
            mk.mk_moe_combine(p0.logits, p0.topk, p0.offsets, p0.perm, w.expert_begin, w.L, p0.Y, Yp, cout, cws,
                              stream=stream, check=False)

        _, ck = timed(combine, 10, 3, stream)
        cbytes = w.T * w.k * w.F * 2 + w.T * w.F * 2 + w.T * w.E * 4 + 3 * w.T * w.k * 4
        r["combine_ms"] = ck
        r["combine_gbs"] = cbytes / ck / 1e6
        r["combine_hbm_frac"] = cbytes / ck / 1e6 / PEAK_HBM_GBS
        del Yp
        # the gate GEMM before routing: logits = X @ W_gate (T x H x E, fp32 out)
        Wg = torch.from_numpy(wl.moe_gate_weights(w, seed=args.seed).view(np.int16)).cuda().view(torch.bfloat16)
        glog = torch.empty(w.T, w.E, dtype=torch.float32, device="cuda")
        gws = mk.workspace(mk.mk_moe_gate_workspace(w.T, w.H, w.E))

        def gate(i):
            mk.mk_moe_gate(p0.X, Wg, glog, gws, stream=stream, check=False)

        _, gk = timed(gate, 20, 5, stream)
        gflops = 2.0 * w.T * w.H * w.E
        gbytes = w.T * w.H * 2 + w.H * w.E * 2 + w.T * w.E * 4
        r["gate_ms"] = gk
        r["gate_tflops"] = gflops / gk / 1e9
        r["gate_gbs"] = gbytes / gk / 1e6
        r["gate_roofline"] = dict(bound="hbm", achieved=round(gbytes / gk / 1e6, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                                  frac=round(gbytes / gk / 1e6 / PEAK_HBM_GBS, 4), traffic=None,
                                  mfma_frac=round(gflops / gk / 1e9 / PEAK_BF16_TFLOPS, 4))
        del Wg, glog, gws
        for tag, kw in [("copy_only", dict(mode=2)), ("gemm_only", dict(mode=3)),
                        ("n_copy128", dict(n_copy=128)), ("xcd_queues", dict(queue_mode=1)),
                        ("expert_order", dict(queue_mode=2)), ("hold", dict(queue_mode=3)),
                        ("tile_128x256dma", dict(tile=mk.TILE_128x256_DMA))]:
            lv = mk.make_launch(**kw)
            _, vk = timed(lambda i: probs[i % copies].run(launch=lv, stream=stream, check=False), 5, 2, stream)
            r[f"variant_{tag}_ms"] = vk
        tc, tg = r["variant_copy_only_ms"], r["variant_gemm_only_ms"]
        # the GEMM kernel alone reads the landing rows cold (evicted from the
        # last-level cache since they were written), so tc + tg overstates
        # the unfused sequence, where the GEMM follows its permute kernel
        r["overlap_eff"] = (tc + tg - kern) / min(tc, tg)
        r["overlap_eff_vs_unfused"] = (uk - kern) / tc
    return r


def bench_ring(args, stream, extra=True):
    """Ring attention, rank 0's share: its queries against all R shards of
    keys and values, the peers' shards moved into the receive buffers by the
    kernel's copy workgroups."""
    import workloads as wl
    from tile_pipelined_gemm_amd import mk
    from tile_pipelined_gemm_amd.harness import RingProblem
    w = wl.CONFIGS["ring"]["make"](args.seed)
    prob = RingProblem(w)
    flops = prob.flops
    H, S, D, R = w.H, w.S, w.D, w.R
    # Q, every shard read once, O written, the R-1 peer shards written to and
    # read back from the receive buffers
    abytes = H * S * D * 2 * (1 + 2 * R + 1 + 2 * 2 * (R - 1))

    def fused(i):
        prob.run(stream=stream, check=False)

    settle(fused, 0.3)
    wall, kern = timed(fused, max(3, args.steps // 2), 2, stream)
    assert mk.mk_poll_status(prob.ws, stream) == mk.MK_OK
    r = dict(workload=wl.CONFIGS["ring"]["desc"], H=H, S=S, D=D, R=R, ms=wall, kernel_ms=kern,
             tflops=flops / kern / 1e9, flops=flops, alg_bytes=abytes,
             mfma_tflops=1.5 * flops / kern / 1e9)
    if extra:
        lau = mk.make_launch(mode=1)
        _, uk = timed(lambda i: prob.run(launch=lau, stream=stream, check=False), 3, 1, stream)
        r["unfused_ms"] = uk
        r["speedup_vs_unfused"] = uk / kern
        for tag, kw in [("n_copy64", dict(n_copy=64))]:
            lv = mk.make_launch(**kw)
            _, vk = timed(lambda i: prob.run(launch=lv, stream=stream, check=False), 3, 1, stream)
            r[f"variant_{tag}_ms"] = vk
    return r


def bench_peaks(stream):
    """Rates measured on this device (mk_peak_*): an MFMA-only bf16 loop on
    every CU with the average engine clock during it, an HBM read stream and
    an HBM copy.  Reported beside the published peaks (which stay the roofline
    denominators)."""
    import torch
    from tile_pipelined_gemm_amd import mk
    ws = mk.workspace(mk.load().mk_peak_workspace())
    khz = mk.mk_wall_clock_khz()
    iters = 4096
    state = {}

    def mfma(i):
        state["f"], state["n"] = mk.mk_peak_mfma(iters, ws, stream=stream)

    settle(mfma, 0.3)
    _, mk_ms = timed(mfma, 10, 3, stream)
    ck = ws[256:256 + 16 * state["n"]].view(torch.int64).cpu().numpy().reshape(-1, 2)
    clock_ghz = float(ck[:, 0].sum()) / float(ck[:, 1].sum()) * khz / 1e6
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    moved = {}

    def rd(i):
        moved["r"] = mk.mk_peak_hbm(src, None, 0, ws, stream=stream)

    _, rd_ms = timed(rd, 10, 3, stream)
    half = src[:2 << 30]
    dst = src[2 << 30:]

    def cp(i):
        moved["c"] = mk.mk_peak_hbm(half, dst, 1, ws, stream=stream)

    _, cp_ms = timed(cp, 10, 3, stream)
    del src, half, dst
    return dict(mfma_bf16_tflops=state["f"] / mk_ms / 1e9, mfma_loop_clock_ghz=clock_ghz,
                mfma_frac_of_published=state["f"] / mk_ms / 1e9 / PEAK_BF16_TFLOPS,
                hbm_read_gbs=moved["r"] / rd_ms / 1e6, hbm_copy_gbs=moved["c"] / cp_ms / 1e6,
                published_bf16_tflops=PEAK_BF16_TFLOPS, published_hbm_gbs=PEAK_HBM_GBS)


def roofline(name, r, peaks):
    """Roofline object of workload `name` from its result r: algorithmic work
    per launch over the mean launch time, against the published peak (and the
    measured one), with the counter-measured HBM traffic when the committed
    summary was taken on the current kernel sources."""
    bound, sources, summary = ROOFLINES[name]
    if bound == "mfma":
        achieved, peak, unit = r["flops"] / r["kernel_ms"] / 1e9, PEAK_BF16_TFLOPS, "TFLOP/s"
        measured = peaks.get("mfma_bf16_tflops") if peaks else None
    else:
        achieved, peak, unit = r["alg_bytes"] / r["kernel_ms"] / 1e6, PEAK_HBM_GBS, "GB/s"
        measured = peaks.get("hbm_read_gbs") if peaks else None
    out = dict(bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit, frac=round(achieved / peak, 4),
               traffic=counter_traffic(sources, summary))
    if measured:
        out["frac_of_measured_peak"] = round(achieved / measured, 4)
    return out


def cpu_baseline(seed):
    """The oracle (numpy float64) timed on whole calls of the AG workload."""
    import numpy as np
    import oracle.ag_gemm as og
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        cores = max((i.get("num_threads", 0) for i in threadpool_info()), default=0) or os.cpu_count()
    except Exception:
        cores = os.cpu_count()
    w = wl.CONFIGS["ag"]["make"](seed)
    flops = 2.0 * w.M * w.K * w.N
    reps, t0 = 0, time.perf_counter()
    while True:                     # whole oracle calls, about 10 s in total
        og.ag_gemm(w.shards, w.B, w.out_dtype, order=w.order, delay_ns=w.delay_ns, unit_rows=w.unit_rows)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 50:
            break
    return dict(value=flops * reps / dt / 1e12, unit="TFLOP/s", cores=int(cores), kind="oracle",
                sample=f"{reps} full oracle calls of the AG workload (gather, float64 GEMM "
                       f"{w.M}x{w.K}x{w.N}, bf16 rounding) in {dt:.1f} s")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the kernels compute one GPU share and there is no multi-GPU launcher.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from tile_pipelined_gemm_amd import mk
    mk.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    if args.ag_timeline:
        import workloads as wl
        from tile_pipelined_gemm_amd.harness import AgProblem, ag_timeline
        prob = AgProblem(wl.CONFIGS["ag"]["make"](seed=args.seed))
        for spec in args.ag_timeline.split(";"):
            kw = {k: int(v) for k, v in (kv.split("=") for kv in spec.split(",") if kv)}
            for _ in range(3):                       # warm up
                prob.run(launch=mk.make_launch(**kw))
            torch.cuda.synchronize()
            print(json.dumps({"launch": spec, **ag_timeline(prob, **kw)}), flush=True)
        return
    if args.moe_timeline:
        import workloads as wl
        from tile_pipelined_gemm_amd.harness import MoeProblem, moe_timeline
        prob = MoeProblem(wl.CONFIGS["moe"]["make"](seed=args.seed))
        for spec in args.moe_timeline.split(";"):
            kw = {k: int(v) for k, v in (kv.split("=") for kv in spec.split(",") if kv)}
            for _ in range(3):                       # warm up
                prob.run(launch=mk.make_launch(**kw))
            torch.cuda.synchronize()
            print(json.dumps({"launch": spec, **moe_timeline(prob, **kw)}), flush=True)
        return
    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        wall, kern = timed(lambda i: dst.copy_(src), args.steps, args.warmup, stream)
        print(json.dumps({"copy_bytes": n, "kernel_ms": kern, "gbs": 2 * n / kern / 1e6}), flush=True)
        return
    only = set(x for x in args.only.split(",") if x)

    def want(x):
        return not only or x in only

    extra = not args.no_extra
    configs = {}
    primary = None
    if want("ag"):
        log("bench: ag")
        primary = bench_ag("ag", args, stream, extra)
        configs["ag"] = primary
    if want("skinny_ag"):
        log("bench: skinny_ag")
        configs["skinny_ag"] = bench_ag("skinny_ag", args, stream, extra)
    if want("rs"):
        log("bench: rs")
        configs["rs"] = bench_rs(args, stream, extra)
    if want("ar"):
        log("bench: ar")
        configs["ar"] = bench_ar(args, stream, extra)
    if want("moe"):
        log("bench: moe")
        configs["moe"] = bench_moe(args, stream, extra)
    if want("ring"):
        log("bench: ring")
        configs["ring"] = bench_ring(args, stream, extra)
    peaks = None
    if not args.no_peaks:
        log("bench: peaks")
        peaks = bench_peaks(stream)
    for k, v in configs.items():
        if k in ROOFLINES:
            v["roofline"] = roofline(k, v, peaks)
        if k == "moe" and "combine_gbs" in v:
            v["combine_roofline"] = dict(bound="hbm", achieved=round(v["combine_gbs"], 2), peak=PEAK_HBM_GBS,
                                         unit="GB/s", frac=round(v["combine_gbs"] / PEAK_HBM_GBS, 4), traffic=None)
    cpu = None
    if primary is not None and not args.no_cpu:
        log("bench: cpu baseline")
        cpu = cpu_baseline(args.seed)
    if primary is None:
        primary = next(iter(configs.values()))
    value = primary["flops"] / primary["ms"] / 1e9
    # counters were taken on the default launch of the AG workload only
    traffic = counter_traffic(AG_KERNEL_SOURCES, AG_COUNTERS) \
        if primary is configs.get("ag") and not args.ag_launch else None
    out = {
        "metric": "fused AG+GEMM / GEMM+RS TFLOP/s at 1 MI355X; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(primary["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": primary["workload"], "M": primary.get("M"), "K": primary.get("K"),
                   "N": primary.get("N"), "R": primary.get("R"), "parallelism": "single GPU share"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(primary["flops"] / primary["kernel_ms"] / 1e9, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(primary["flops"] / primary["kernel_ms"] / 1e9 / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "peaks_measured": {k: round(v, 4) for k, v in peaks.items()} if peaks else None,
        "configs": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in configs.items()},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
