"""MoE gate GEMM oracle (the step before routing).

Test infrastructure: only tests/, the package smoke check and bench.py's CPU
baseline use this module; the HIP library never does.

[P1] "Los cinco núcleos fusionados", row "Envío MoE + GEMM", and explainer
slide "04 / 07 — Granos": tokens are routed to the ranks of their experts.
The pages start from the routing; the scores it ranks come from the gate, a
linear map of each token's hidden state to one logit per expert.

Readings (the pages fix none of these):
* logits = X @ W_gate with X [T x H] and W_gate [H x E] bf16 (row-major,
  W_gate's column e is expert e's gate vector), accumulated exactly here in
  float64 and rounded once to float32, the dtype routing consumes.
* No bias, no softmax, no noise: routing ranks the raw logits.
"""
import numpy as np

from .numerics import bf16_to_f64


def gate_logits(X, W_gate):
    """Return (logits64 [T x E], logits32): the float64 product and its float32 rounding."""
    L64 = bf16_to_f64(X) @ bf16_to_f64(W_gate)
    return L64, L64.astype(np.float32)
