"""CPU oracle for the tile-pipelined fused GEMM kernels (test infrastructure only).

This package is a plain, slow, obviously correct float64 restatement of what
the fused kernels compute.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does, and
it shares no code with the HIP library (the only common module is the seeded
input generator in ``workloads``, which holds no arithmetic of the method).

Sources (the web pages describing mKernel; cited by title and section):

* [P1] "Conozca mKernel, una biblioteca de núcleo fusionado con múltiples GPU y
  múltiples nodos para comunicación impulsada por GPU" (7minutos.es), sections
  "Los cinco núcleos fusionados" (five-kernel table) and the visual explainer
  slide "04 / 07 — Granos".
* [P3] the Arabic translation of the same article (k7ail.com, "تعرف على mKernel"),
  table "الحبات الخمس المنصهرة" (the five fused kernels), whose cells are the
  cleanest copy of the same table.

What the pages fix: AllGather+GEMM computes C = A @ B where every rank holds a
shard of A and the local GEMM consumes tiles as the gathered shards arrive;
GEMM+ReduceScatter computes C = A @ B and each finished output tile is reduced
and sent to the rank that owns it; GEMM+AllReduce computes the same sum and
leaves all of it on every rank; Ring Attention rotates key/value shards round
the ring while attention consumes them; MoE dispatch+GEMM routes tokens to expert
ranks and runs the per-expert grouped GEMM on the tokens as they land.  The
pages give no dtypes, layouts, tie-breaks or worked numbers; every such choice
made here is a reading, listed in each module's docstring.

Pinning: every function is checked by ``tests/test_oracle_*.py`` against
brute force (``math.fsum`` of exact products), closed forms (identity and
one-hot operands), exact integer arithmetic, invariants (arrival-order
independence, reduce-scatter over all owners = all-reduce, dispatch is a
permutation whose counts sum to T*k) and library special cases.
"""
from . import numerics, schedule, ag_gemm, gemm_rs, gemm_ar, moe, moe_combine, ring_attn  # noqa: F401
