"""Device-side problem holders for the three fused operations.

Each class uploads one seeded workload (``workloads``) into device memory
once, owns the outputs and the workspace, and runs the operation through the
C-ABI binding.  PyTorch only provides device memory and streams here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import mk


def bf16_tensor(u16: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(u16, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def f32_tensor(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_numpy(t: torch.Tensor) -> np.ndarray:
    """bf16 -> uint16 bit patterns, float32 -> float32, int32 -> int32."""
    if t.dtype == torch.bfloat16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


def _out_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


class AgProblem:
    def __init__(self, w, device="cuda"):
        self.w = w
        self.shards = [bf16_tensor(s, device) for s in w.shards]
        self.B = bf16_tensor(w.B, device)
        self.C = torch.empty(w.M, w.N, dtype=_out_dtype(w.out_dtype), device=device)
        self.Ag = torch.empty(w.M, w.K, dtype=torch.bfloat16, device=device)
        self.ws = mk.workspace(mk.mk_ag_gemm_workspace(w.R, w.m_shard, w.K, w.N, w.unit_rows), device)

    @property
    def flops(self):
        return 2.0 * self.w.M * self.w.N * self.w.K

    def run(self, launch=None, order=None, delay_ns=None, withhold=-1, stream=None, check=True):
        order = self.w.order if order is None else order
        delay_ns = self.w.delay_ns if delay_ns is None else delay_ns
        return mk.mk_ag_gemm(self.shards, self.B, self.C, self.Ag, self.ws, order=order, delay_ns=delay_ns,
                             unit_rows=self.w.unit_rows, withhold=withhold, launch=launch, stream=stream,
                             check=check)

    def output(self):
        return to_numpy(self.C)


class RsProblem:
    def __init__(self, w, device="cuda", landing=False):
        self.w = w
        self.A = bf16_tensor(w.A, device)
        self.B = bf16_tensor(w.B, device)
        self.P = [f32_tensor(p, device) for p in w.partials]
        mb = w.M // w.R
        self.out = [torch.empty(mb, w.N, dtype=_out_dtype(w.out_dtype), device=device) for _ in range(w.R)]
        code = mk.MK_BF16 if w.out_dtype == "bf16" else mk.MK_F32
        self.ws = mk.workspace(mk.mk_gemm_rs_workspace(w.M, w.K, w.N, w.R, code), device)
        # landing buffers for the partial sums the copy workgroups move
        self.landing = [torch.empty_like(p) for p in self.P] if landing else None

    @property
    def flops(self):
        return 2.0 * self.w.M * self.w.N * self.w.K

    def _sched(self, arrival, order, delay_ns):
        """The workload's arrival schedule (or the given order/delays) when
        arrival is True and the workload has one, else none."""
        if not arrival or self.w.unit_rows is None:
            return dict()
        return dict(order=self.w.order if order is None else order,
                    delay_ns=self.w.delay_ns if delay_ns is None else delay_ns, unit_rows=self.w.unit_rows)

    def run(self, launch=None, stream=None, check=True, arrival=True, order=None, delay_ns=None, withhold=-1):
        return mk.mk_gemm_rs(self.A, self.B, self.P, self.out, self.ws, launch=launch, stream=stream, check=check,
                             withhold=withhold, landing=self.landing if arrival else None,
                             **self._sched(arrival, order, delay_ns))

    def output(self):
        return np.vstack([to_numpy(o) for o in self.out])


class ArProblem:
    """GEMM -> AllReduce on an RsWorkload: every rank's output is the whole S."""

    def __init__(self, w, device="cuda", landing=False):
        self.w = w
        self.A = bf16_tensor(w.A, device)
        self.B = bf16_tensor(w.B, device)
        self.P = [f32_tensor(p, device) for p in w.partials]
        self.out = [torch.empty(w.M, w.N, dtype=_out_dtype(w.out_dtype), device=device) for _ in range(w.R)]
        code = mk.MK_BF16 if w.out_dtype == "bf16" else mk.MK_F32
        self.ws = mk.workspace(mk.mk_gemm_ar_workspace(w.M, w.K, w.N, w.R, code), device)
        self.landing = [torch.empty_like(p) for p in self.P] if landing else None

    @property
    def flops(self):
        return 2.0 * self.w.M * self.w.N * self.w.K

    _sched = RsProblem._sched

    def run(self, launch=None, stream=None, check=True, arrival=True, order=None, delay_ns=None, withhold=-1):
        return mk.mk_gemm_ar(self.A, self.B, self.P, self.out, self.ws, launch=launch, stream=stream, check=check,
                             withhold=withhold, landing=self.landing if arrival else None,
                             **self._sched(arrival, order, delay_ns))

    def outputs(self):
        return [to_numpy(o) for o in self.out]


class MoeProblem:
    def __init__(self, w, device="cuda"):
        self.w = w
        self.X = bf16_tensor(w.X, device)
        self.logits = f32_tensor(w.logits, device)
        self.W = [bf16_tensor(x, device) for x in w.W]
        cap = w.T * min(w.k, w.L)
        i32 = dict(dtype=torch.int32, device=device)
        self.topk = torch.empty(w.T, w.k, **i32)
        self.counts = torch.empty(w.E, **i32)
        self.offsets = torch.empty(w.E + 1, **i32)
        self.perm = torch.empty(w.T * w.k, **i32)
        self.n_local = torch.empty(1, **i32)
        self.Xs = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=device)   # receive buffer: row t = token t
        self.Y = torch.empty(cap, w.F, dtype=_out_dtype(w.out_dtype), device=device)
        self.ws = mk.workspace(mk.mk_moe_dispatch_gemm_workspace(w.T, w.H, w.E, w.k, w.L, w.F), device)

    def run(self, launch=None, order=None, delay_ns=None, withhold=-1, stream=None, check=True):
        order = self.w.order if order is None else order
        delay_ns = self.w.delay_ns if delay_ns is None else delay_ns
        return mk.mk_moe_dispatch_gemm(self.X, self.logits, self.W, self.w.k, self.w.expert_begin, self.topk,
                                       self.counts, self.offsets, self.perm, self.n_local, self.Xs, self.Y,
                                       self.ws, order=order, delay_ns=delay_ns, block_tokens=self.w.block_tokens,
                                       withhold=withhold, launch=launch, stream=stream, check=check)

    def local_rows(self) -> int:
        return int(self.n_local.item())

    def received_rows(self) -> int:
        """Tokens with at least one local expert (the rows of Xs written)."""
        lo = int(self.offsets[self.w.expert_begin].item())
        hi = int(self.offsets[self.w.expert_begin + self.w.L].item())
        return int(torch.unique(self.perm[lo:hi] // self.w.k).numel())

    def flops(self) -> float:
        return 2.0 * self.local_rows() * self.w.H * self.w.F

    def outputs(self):
        n = self.local_rows()
        return dict(topk=to_numpy(self.topk), counts=to_numpy(self.counts), offsets=to_numpy(self.offsets),
                    perm=to_numpy(self.perm), n_local=n, Y=to_numpy(self.Y[:n]))


class RingProblem:
    """Ring attention: rank 0's queries, every rank's key/value shard and the
    receive buffers the ring fills."""

    def __init__(self, w, device="cuda"):
        self.w = w
        self.Q = bf16_tensor(w.Q, device)
        self.K = [bf16_tensor(k, device) for k in w.K]
        self.V = [bf16_tensor(v, device) for v in w.V]
        self.O = torch.empty(w.H, w.S, w.D, dtype=_out_dtype(w.out_dtype), device=device)
        if w.R > 1:
            self.Kr = torch.empty(w.R - 1, w.H, w.S, w.D, dtype=torch.bfloat16, device=device)
            self.Vr = torch.empty_like(self.Kr)
        else:
            self.Kr = self.Vr = None
        self.ws = mk.workspace(mk.mk_ring_attn_workspace(w.H, w.S, w.R), device)

    @property
    def flops(self):
        """Q K^T and P V: 4 * H * S * (R*S) * D."""
        w = self.w
        return 4.0 * w.H * w.S * (w.R * w.S) * w.D

    def run(self, launch=None, order=None, delay_ns=None, withhold=-1, stream=None, check=True):
        order = self.w.order if order is None else order
        delay_ns = self.w.delay_ns if delay_ns is None else delay_ns
        return mk.mk_ring_attn(self.Q, self.K, self.V, self.O, self.Kr, self.Vr, self.ws, order=order,
                               delay_ns=delay_ns, withhold=withhold, launch=launch, stream=stream, check=check)

    def output(self):
        return to_numpy(self.O)


def ag_timeline(prob, **launch_kw):
    """Run one AG+GEMM call with the tile and copy logs on and summarise its
    timeline (microseconds from the first logged event)."""
    import numpy as np
    n_rec = 8 * max(4096, 2 * mk.MK_MAX_UNITS * 64)
    tlog = torch.full((n_rec,), -1, dtype=torch.int32, device="cuda")
    clog = torch.full((n_rec,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=mk.make_launch(tile_log=tlog, copy_log=clog, **launch_kw))
    torch.cuda.synchronize()
    khz = mk.load().mk_wall_clock_khz()
    T = tlog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    Cl = clog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    T = T[T[:, 0] >= 0]
    Cl = Cl[Cl[:, 0] >= 0]
    stamps = np.concatenate([T[:, 5:8].ravel(), Cl[:, 3:5].ravel()]) & 0xffffffff
    base = int(stamps.min())
    us = lambda x: ((np.asarray(x) - base) & 0xffffffff) * 1000.0 / khz
    out = {"tiles": int(len(T)), "copy_items": int(len(Cl))}
    if len(Cl):
        land = {}
        for u, _, _, _, te in Cl[:, :5]:
            land[int(u)] = max(land.get(int(u), 0.0), float(us(te)))
        out.update(copy_first_start_us=float(us(Cl[:, 3]).min()), copy_last_end_us=float(us(Cl[:, 4]).max()),
                   copy_item_mean_us=float((us(Cl[:, 4]) - us(Cl[:, 3])).mean()),
                   copy_workgroups=int(len(set(Cl[:, 2].tolist()))),
                   unit_land_us=[round(land[u], 2) for u in sorted(land)])
    if len(T):
        wait = us(T[:, 6]) - us(T[:, 5])
        comp = us(T[:, 7]) - us(T[:, 6])
        out.update(first_tile_ready_us=float(us(T[:, 6]).min()), last_tile_done_us=float(us(T[:, 7]).max()),
                   tile_wait_mean_us=float(wait.mean()), tile_wait_max_us=float(wait.max()),
                   tile_compute_mean_us=float(comp.mean()), tile_compute_max_us=float(comp.max()),
                   compute_workgroups=int(len(set(T[:, 4].tolist()))))
    return out


def moe_timeline(prob, **launch_kw):
    """Run one MoE dispatch + grouped GEMM call with the tile and copy logs on
    and summarise its timeline (microseconds from the first logged event)."""
    import numpy as np
    w = prob.w
    n_tiles = (w.T * min(w.k, w.L) // 128 + w.L + 1) * ((w.F + 127) // 128)
    n_items = w.T + w.block_tokens
    tlog = torch.full((8 * n_tiles,), -1, dtype=torch.int32, device="cuda")
    clog = torch.full((8 * n_items,), -1, dtype=torch.int32, device="cuda")
    prob.run(launch=mk.make_launch(tile_log=tlog, copy_log=clog, **launch_kw))
    torch.cuda.synchronize()
    khz = mk.load().mk_wall_clock_khz()
    T = tlog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    Cl = clog.cpu().numpy().reshape(-1, 8).astype(np.int64)
    T = T[T[:, 0] >= 0]
    Cl = Cl[Cl[:, 0] >= 0]
    stamps = np.concatenate([T[:, 5:8].ravel(), Cl[:, 3:5].ravel()]) & 0xffffffff
    base = int(stamps.min())
    us = lambda x: ((np.asarray(x) - base) & 0xffffffff) * 1000.0 / khz
    out = {"tiles": int(len(T)), "copy_items": int(len(Cl))}
    if len(Cl):
        out.update(copy_first_start_us=float(us(Cl[:, 3]).min()), copy_last_end_us=float(us(Cl[:, 4]).max()),
                   copy_item_mean_us=float((us(Cl[:, 4]) - us(Cl[:, 3])).mean()),
                   copy_index_mean_us=float((us(Cl[:, 6]) - us(Cl[:, 3])).mean()),
                   copy_rows_mean_us=float((us(Cl[:, 7]) - us(Cl[:, 6])).mean()),
                   copy_release_mean_us=float((us(Cl[:, 4]) - us(Cl[:, 7])).mean()),
                   copy_rows_per_item=float(Cl[:, 5].mean()),
                   copy_workgroups=int(len(set(Cl[:, 2].tolist()))))
    if len(T):
        take, ready, done = us(T[:, 5]), us(T[:, 6]), us(T[:, 7])
        comp = done - ready
        per_wg = {}
        for wg, d in zip(T[:, 4].tolist(), done.tolist()):
            per_wg[wg] = max(per_wg.get(wg, 0.0), d)
        ends = np.array(sorted(per_wg.values()))
        out.update(first_tile_ready_us=float(ready.min()), last_tile_done_us=float(done.max()),
                   tile_wait_mean_us=float((ready - take).mean()), tile_wait_max_us=float((ready - take).max()),
                   tile_compute_mean_us=float(comp.mean()), tile_compute_p10_us=float(np.percentile(comp, 10)),
                   tile_compute_p90_us=float(np.percentile(comp, 90)),
                   tiles_per_workgroup_max=int(np.bincount(T[:, 4]).max()),
                   compute_workgroups=int(len(per_wg)),
                   workgroup_end_p10_us=float(np.percentile(ends, 10)),
                   workgroup_end_p50_us=float(np.percentile(ends, 50)))
    return out
