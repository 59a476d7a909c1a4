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
    def __init__(self, w, device="cuda"):
        self.w = w
        self.A = bf16_tensor(w.A, device)
        self.B = bf16_tensor(w.B, device)
        self.P = [f32_tensor(p, device) for p in w.partials]
        mb = w.M // w.R
        self.out = [torch.empty(mb, w.N, dtype=_out_dtype(w.out_dtype), device=device) for _ in range(w.R)]
        code = mk.MK_BF16 if w.out_dtype == "bf16" else mk.MK_F32
        self.ws = mk.workspace(mk.mk_gemm_rs_workspace(w.M, w.K, w.N, w.R, code), device)

    @property
    def flops(self):
        return 2.0 * self.w.M * self.w.N * self.w.K

    def run(self, launch=None, stream=None, check=True):
        return mk.mk_gemm_rs(self.A, self.B, self.P, self.out, self.ws, launch=launch, stream=stream, check=check)

    def output(self):
        return np.vstack([to_numpy(o) for o in self.out])


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
        self.Xs = torch.empty(cap, w.H, dtype=torch.bfloat16, device=device)
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

    def flops(self) -> float:
        return 2.0 * self.local_rows() * self.w.H * self.w.F

    def outputs(self):
        n = self.local_rows()
        return dict(topk=to_numpy(self.topk), counts=to_numpy(self.counts), offsets=to_numpy(self.offsets),
                    perm=to_numpy(self.perm), n_local=n, Y=to_numpy(self.Y[:n]))
