"""Oracle results for the full-size workloads, computed once per test session.

Whole outputs of the benchmark-size workloads are compared element by element
against these (the float64 oracle takes seconds per workload on the host's
cores), and the GEMM+ReduceScatter and GEMM+AllReduce tests share one
reduced sum.
"""
import functools

import oracle.ag_gemm as og
import oracle.gemm_rs as orc
import workloads as wl


@functools.lru_cache(maxsize=2)
def ag_product(name):
    """float64 C of the full-size AllGather+GEMM workload `name` ("ag" or
    "skinny_ag"), with the workload."""
    w = wl.CONFIGS[name]["make"]()
    C64, _ = og.ag_gemm(w.shards, w.B, w.out_dtype)
    return w, C64


@functools.lru_cache(maxsize=1)
def rs_workload():
    return wl.CONFIGS["rs"]["make"]()


@functools.lru_cache(maxsize=1)
def rs_reduced_sum():
    """float64 S = A @ B + P_1 + ... + P_7 of the full-size GEMM+RS workload."""
    w = rs_workload()
    S, _, _ = orc.gemm_rs(w.A, w.B, w.partials, w.R)
    return S
