"""Seeded synthetic workloads shared by the oracle, the tests and the benchmark.

This module only draws random numbers and packages them: it holds none of the
arithmetic of the fused operations (no products, sums, routing or dispatch).
Both the HIP path and the CPU oracle consume the arrays produced here, bit for
bit, so that neither side regenerates or re-rounds the other's inputs.

Random-number recipe
--------------------
* Generator: numpy PCG64. ``SeedSequence(seed).spawn(n)`` gives one independent
  stream per tensor, in the fixed order in which each ``make_*`` function
  lists its tensors.
* Real-valued tensors are sampled in float32 and rounded to bfloat16 with
  round-to-nearest-even (``f32_to_bf16_bits``).  ``N(0, v)`` means variance ``v``
  (standard deviation ``sqrt(v)``), which keeps GEMM outputs at about unit
  variance.
* bfloat16 tensors are carried as ``uint16`` bit patterns.
* Arrival schedules are a seeded permutation of the delivery units plus a
  per-unit release delay in nanoseconds (uniform, integer).
* MoE logits follow a Zipf(s) expert popularity: ``logit[t, e] = -s*ln(e+1) +
  g[t, e]`` with ``g`` standard Gumbel noise, formed in float64 and stored as
  float32.  Taking the top-k of such logits draws k distinct experts per token
  with probability proportional to ``(e+1)^-s`` (the Gumbel-top-k trick).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "AgWorkload", "RsWorkload", "MoeWorkload", "CONFIGS",
    "make_ag", "make_rs", "make_moe", "moe_combine_inputs", "moe_gate_weights", "make_ring", "fingerprint",
]


# ---------------------------------------------------------------------------
# input quantisation
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction here, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    z = rng.standard_normal(shape, dtype=np.float32)
    if var != 1.0:
        z *= np.float32(np.sqrt(var))
    return f32_to_bf16_bits(z)


def _uniform_bf16(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    z = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return f32_to_bf16_bits(z)


def _streams(seed: int, n: int) -> List[np.random.Generator]:
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def fingerprint(a: np.ndarray) -> str:
    """sha256 of the raw bytes (first 16 hex digits) for reproducibility records."""
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# workload descriptions
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class AgWorkload:
    """AllGather -> GEMM: R shards of A (each m_shard x K) and B (K x N)."""
    shards: List[np.ndarray]        # R x uint16[m_shard, K]
    B: np.ndarray                   # uint16[K, N]
    order: np.ndarray               # int32[n_units], permutation: issue order of units
    delay_ns: np.ndarray            # uint32[n_units], earliest release of unit c after start
    unit_rows: int                  # rows of the gathered A per delivery unit
    out_dtype: str                  # "bf16" | "f32"

    @property
    def R(self): return len(self.shards)
    @property
    def m_shard(self): return self.shards[0].shape[0]
    @property
    def K(self): return self.B.shape[0]
    @property
    def N(self): return self.B.shape[1]
    @property
    def M(self): return self.R * self.m_shard


@dataclasses.dataclass
class RsWorkload:
    """GEMM -> ReduceScatter: A (M x K), B (K x N), R-1 resident fp32 partials (M x N).

    Optional arrival schedule of the partial sums: unit u = (p - 1) * (M /
    unit_rows) + b is rows [b * unit_rows, (b + 1) * unit_rows) of partial p
    (p = 1..R-1); ``order`` is a permutation of the units, ``delay_ns`` their
    release times.  ``unit_rows`` None: every partial resident from the start.
    """
    A: np.ndarray                   # uint16[M, K]
    B: np.ndarray                   # uint16[K, N]
    partials: List[np.ndarray]      # (R-1) x float32[M, N]
    R: int
    out_dtype: str
    order: Optional[np.ndarray] = None      # int32[(R-1) * M / unit_rows]
    delay_ns: Optional[np.ndarray] = None   # uint32[(R-1) * M / unit_rows]
    unit_rows: Optional[int] = None

    @property
    def M(self): return self.A.shape[0]
    @property
    def K(self): return self.A.shape[1]
    @property
    def N(self): return self.B.shape[1]


@dataclasses.dataclass
class MoeWorkload:
    """MoE dispatch -> grouped GEMM over the L local experts [expert_begin, expert_begin+L)."""
    X: np.ndarray                   # uint16[T, H]
    logits: np.ndarray              # float32[T, E]
    W: List[np.ndarray]             # L x uint16[H, F]
    k: int
    expert_begin: int
    order: np.ndarray               # int32[n_blocks], arrival order of token blocks
    delay_ns: np.ndarray            # uint32[n_blocks]
    block_tokens: int
    out_dtype: str

    @property
    def T(self): return self.X.shape[0]
    @property
    def H(self): return self.X.shape[1]
    @property
    def E(self): return self.logits.shape[1]
    @property
    def L(self): return len(self.W)
    @property
    def F(self): return self.W[0].shape[1]


@dataclasses.dataclass
class RingWorkload:
    """Ring attention: rank 0's queries and every rank's key/value shard."""
    Q: np.ndarray                   # uint16[H, S, D]
    K: List[np.ndarray]             # R x uint16[H, S, D], rank r's keys
    V: List[np.ndarray]             # R x uint16[H, S, D]
    order: np.ndarray               # int32[(R-1)*H], arrival order of units (ring step s >= 1, head h): (s-1)*H + h
    delay_ns: np.ndarray            # uint32[(R-1)*H]
    out_dtype: str

    @property
    def H(self): return self.Q.shape[0]
    @property
    def S(self): return self.Q.shape[1]
    @property
    def D(self): return self.Q.shape[2]
    @property
    def R(self): return len(self.K)


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------
def make_ag(R: int, m_shard: int, K: int, N: int, *, seed: int = 0, dist: str = "normal",
            b_var: Optional[float] = None, unit_rows: Optional[int] = None,
            max_delay_ns: int = 0, out_dtype: str = "bf16") -> AgWorkload:
    """AllGather->GEMM inputs.

    dist="normal": A ~ N(0,1), B ~ N(0, b_var) (default 1/K).
    dist="uniform": A, B ~ U[-1, 1].
    dist="int": A, B uniform integers in {-2..2} (exact in fp32 accumulation).
    Stream order: schedule, B, shard 0..R-1.
    """
    unit_rows = unit_rows or m_shard
    M = R * m_shard
    if M % unit_rows:
        raise ValueError("unit_rows must divide the gathered row count")
    n_units = M // unit_rows
    st = _streams(seed, 2 + R)
    order = st[0].permutation(n_units).astype(np.int32)
    if max_delay_ns > 0:
        delay = st[0].integers(0, max_delay_ns, size=n_units, endpoint=True).astype(np.uint32)
    else:
        delay = np.zeros(n_units, np.uint32)
    if dist == "normal":
        B = _normal_bf16(st[1], (K, N), b_var if b_var is not None else 1.0 / K)
        shards = [_normal_bf16(st[2 + r], (m_shard, K), 1.0) for r in range(R)]
    elif dist == "uniform":
        B = _uniform_bf16(st[1], (K, N), -1.0, 1.0)
        shards = [_uniform_bf16(st[2 + r], (m_shard, K), -1.0, 1.0) for r in range(R)]
    elif dist == "int":
        B = f32_to_bf16_bits(st[1].integers(-2, 2, size=(K, N), endpoint=True).astype(np.float32))
        shards = [f32_to_bf16_bits(st[2 + r].integers(-2, 2, size=(m_shard, K), endpoint=True)
                                   .astype(np.float32)) for r in range(R)]
    else:
        raise ValueError(dist)
    return AgWorkload(shards, B, order, delay, unit_rows, out_dtype)


def make_rs(M: int, K: int, N: int, R: int, *, seed: int = 0, dist: str = "normal",
            out_dtype: str = "f32", unit_rows: Optional[int] = None, max_delay_ns: int = 0) -> RsWorkload:
    """GEMM->ReduceScatter inputs. Stream order: A, B, partial 1..R-1, schedule.

    unit_rows (optional): the partial sums arrive in units of (peer, row
    block of unit_rows rows), in a seeded order with release delays uniform
    in [0, max_delay_ns]."""
    st = _streams(seed, 2 + (R - 1) + 1)
    if dist == "normal":
        A = _normal_bf16(st[0], (M, K), 1.0)
        B = _normal_bf16(st[1], (K, N), 1.0 / K)
        P = [st[2 + p].standard_normal((M, N), dtype=np.float32) for p in range(R - 1)]
    elif dist == "int":
        A = f32_to_bf16_bits(st[0].integers(-2, 2, size=(M, K), endpoint=True).astype(np.float32))
        B = f32_to_bf16_bits(st[1].integers(-2, 2, size=(K, N), endpoint=True).astype(np.float32))
        P = [st[2 + p].integers(-64, 64, size=(M, N), endpoint=True).astype(np.float32)
             for p in range(R - 1)]
    else:
        raise ValueError(dist)
    if unit_rows is None:
        return RsWorkload(A, B, P, R, out_dtype)
    if M % unit_rows:
        raise ValueError("unit_rows must divide M")
    n_units = (R - 1) * (M // unit_rows)
    sch = st[2 + (R - 1)]
    order = sch.permutation(n_units).astype(np.int32)
    if max_delay_ns > 0:
        delay = sch.integers(0, max_delay_ns, size=n_units, endpoint=True).astype(np.uint32)
    else:
        delay = np.zeros(n_units, np.uint32)
    return RsWorkload(A, B, P, R, out_dtype, order, delay, unit_rows)


def zipf_gumbel_logits(rng: np.random.Generator, T: int, E: int, s: float) -> np.ndarray:
    """Logits whose top-k draws experts without replacement with P(e) ~ (e+1)^-s."""
    u = rng.random((T, E))                      # float64 in [0, 1)
    u = np.maximum(u, np.finfo(np.float64).tiny)
    g = -np.log(-np.log(u))
    base = -s * np.log(np.arange(1, E + 1, dtype=np.float64))
    return (base[None, :] + g).astype(np.float32)


def make_moe(T: int, H: int, E: int, k: int, L: int, F: int, *, seed: int = 0,
             zipf_s: float = 1.1, expert_begin: int = 0, block_tokens: Optional[int] = None,
             logits: Optional[np.ndarray] = None, dist: str = "normal",
             out_dtype: str = "bf16") -> MoeWorkload:
    """MoE dispatch->grouped GEMM inputs. Stream order: schedule, logits, X, W_0..W_{L-1}."""
    block_tokens = block_tokens or T
    if T % block_tokens:
        raise ValueError("block_tokens must divide T")
    n_blocks = T // block_tokens
    st = _streams(seed, 3 + L)
    order = st[0].permutation(n_blocks).astype(np.int32)
    delay = np.zeros(n_blocks, np.uint32)
    if logits is None:
        logits = zipf_gumbel_logits(st[1], T, E, zipf_s)
    if dist == "normal":
        X = _normal_bf16(st[2], (T, H), 1.0)
        W = [_normal_bf16(st[3 + e], (H, F), 1.0 / H) for e in range(L)]
    elif dist == "int":
        X = f32_to_bf16_bits(st[2].integers(-2, 2, size=(T, H), endpoint=True).astype(np.float32))
        W = [f32_to_bf16_bits(st[3 + e].integers(-2, 2, size=(H, F), endpoint=True).astype(np.float32))
             for e in range(L)]
    else:
        raise ValueError(dist)
    return MoeWorkload(X, np.ascontiguousarray(logits, np.float32), W, k, expert_begin,
                       order, delay, block_tokens, out_dtype)


def moe_combine_inputs(w: "MoeWorkload", *, seed: int = 0):
    """Expert outputs for the combine step of MoE workload w: (Y_local
    uint16[T*min(k, L), F], Y_peer uint16[T*k, F]), N(0, 1) in bf16.  Y_local
    stands for the local grouped-GEMM output (capacity rows; the first
    n_local are read); Y_peer for the outputs the other ranks return, one row
    per dispatch position (rows of local positions are not read)."""
    st = _streams(seed + 7919, 2)
    Yl = _normal_bf16(st[0], (w.T * min(w.k, w.L), w.F), 1.0)
    Yp = _normal_bf16(st[1], (w.T * w.k, w.F), 1.0)
    return Yl, Yp


def moe_gate_weights(w: "MoeWorkload", seed: int = 0, dist: str = "normal") -> np.ndarray:
    """Gate weights W_gate [H x E] bf16 for an MoE workload: N(0, 1/H), so the
    logits have about unit variance; dist="int": integers in {-2..2}.
    Its own stream (seed, 9001): the workload's tensors are unchanged."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 9001])))
    H, E = w.X.shape[1], w.logits.shape[1]
    if dist == "int":
        return f32_to_bf16_bits(rng.integers(-2, 2, size=(H, E), endpoint=True).astype(np.float32))
    return _normal_bf16(rng, (H, E), 1.0 / H)


def make_ring(H: int, S: int, D: int, R: int, *, seed: int = 0, step_delay_ns: int = 0,
              out_dtype: str = "bf16") -> RingWorkload:
    """Ring-attention inputs.  Stream order: schedule, Q, K_0..K_{R-1}, V_0..V_{R-1}.

    Q, K, V ~ N(0, 1) in bf16.  Units (ring step s = 1..R-1, head h) arrive
    step by step (a ring delivers step s after step s-1), the heads of one
    step in a seeded order; unit (s, h) is released (s-1)*step_delay_ns after
    the first copy starts.
    """
    st = _streams(seed, 2 + 2 * R)
    order = np.concatenate([(s - 1) * H + st[0].permutation(H) for s in range(1, R)]).astype(np.int32) \
        if R > 1 else np.zeros(0, np.int32)
    delay = np.array([((u // H)) * step_delay_ns for u in range((R - 1) * H)], np.uint32)
    Q = _normal_bf16(st[1], (H, S, D), 1.0)
    K = [_normal_bf16(st[2 + r], (H, S, D), 1.0) for r in range(R)]
    V = [_normal_bf16(st[2 + R + r], (H, S, D), 1.0) for r in range(R)]
    return RingWorkload(Q, K, V, order, delay, out_dtype)


# ---------------------------------------------------------------------------
# the five workloads (shapes of the fused kernels' single-GPU share)
# ---------------------------------------------------------------------------
def _tiny_ag(seed=0):
    return make_ag(4, 64, 128, 96, seed=seed, dist="uniform", out_dtype="f32")


def _ag(seed=0):
    return make_ag(8, 1024, 8192, 3584, seed=seed, unit_rows=128, max_delay_ns=20000,
                   out_dtype="bf16")


def _rs(seed=0):
    return make_rs(8192, 3584, 8192, 8, seed=seed, out_dtype="f32")


def _moe(seed=0):
    return make_moe(4096, 7168, 256, 8, 32, 2048, seed=seed, zipf_s=1.1, block_tokens=512,
                    out_dtype="bf16")


def _ring(seed=0):
    return make_ring(16, 4096, 128, 8, seed=seed)


def _skinny_ag(seed=0):
    return make_ag(8, 16, 8192, 28672, seed=seed, out_dtype="bf16")


CONFIGS: Dict[str, dict] = {
    "tiny_ag": dict(make=_tiny_ag, op="ag", desc="AG+GEMM R=4 x 64x128, N=96, fp32 out"),
    "ag": dict(make=_ag, op="ag", desc="AG+GEMM R=8 x 1024x8192, N=3584, 128-row chunks, 0-20us delays"),
    "rs": dict(make=_rs, op="rs", desc="GEMM+RS 8192x3584x8192, 7 fp32 partials, 8 owners"),
    "moe": dict(make=_moe, op="moe", desc="MoE T=4096 H=7168 top-8 of 256, 32 local experts, F=2048"),
    "skinny_ag": dict(make=_skinny_ag, op="ag", desc="AG+GEMM R=8 x 16x8192, N=28672"),
    "ring": dict(make=_ring, op="ring", desc="Ring attention R=8 x 4096 tokens, 16 heads of 128, non-causal"),
}
