"""Ring Attention oracle (sequence-parallel attention).

Test infrastructure: only tests/, the package smoke check and bench.py's CPU
baseline use this module; the HIP library never does.

[P1] "Los cinco núcleos fusionados", row "Ring Attention" ([P3] table
"الحبات الخمس المنصهرة", same row; the explainer slide "04 / 07" repeats
it): attention is computed in parallel over a sequence split across ranks;
at each step a key/value shard moves one place round the ring while the
local FlashAttention consumes the shard received before it, with compute
and the ring transfers running together in one persistent kernel.

Readings (the pages give no shapes, masks, scales or dtypes):
* Each of R ranks holds S consecutive tokens: queries Q_r and keys/values
  K_r, V_r, each [H][S][D] (H heads, head dimension D).  This GPU is rank 0;
  the other ranks' K/V shards are resident buffers.  After the R steps of
  the ring rank 0 has seen every shard: its output is full (non-causal)
  attention of its queries over all R*S keys,
      O[h, i] = sum_j softmax_j(Q[h, i] . K[h, j] / sqrt(D)) V[h, j].
* Ring order: at step s rank 0 holds the shard of rank (R - s) mod R (its own
  at step 0), the order in which a ring that passes shards to the next rank
  delivers them.  The result does not depend on the order mathematically;
  the kernel accumulates in exactly this order.
* Inputs bf16, exact float64 arithmetic here, output rounded once.
"""
import numpy as np

from .numerics import bf16_to_f64, cast_out


def ring_order(R: int):
    """Shard held by rank 0 at ring step s, s = 0..R-1."""
    return [(R - s) % R for s in range(R)]


def ring_attention(Q, K_shards, V_shards, out_dtype="bf16"):
    """Return (O64 [H][S][D], O in the output dtype).  K_shards[r], V_shards[r]
    are rank r's [H][S][D] key and value shards; Q is rank 0's queries."""
    q = bf16_to_f64(Q)
    K = np.concatenate([bf16_to_f64(k) for k in K_shards], axis=1)   # [H][R*S][D]
    V = np.concatenate([bf16_to_f64(v) for v in V_shards], axis=1)
    D = q.shape[2]
    O = np.empty_like(q)
    for h in range(q.shape[0]):
        s = (q[h] @ K[h].T) / np.sqrt(D)
        s -= s.max(axis=1, keepdims=True)          # the shift cancels in the ratio below
        p = np.exp(s)
        O[h] = (p @ V[h]) / p.sum(axis=1, keepdims=True)
    return O, cast_out(O, out_dtype)


def ring_attention_rows(Q, K_shards, V_shards, h: int, rows):
    """float64 outputs of head h for the query rows `rows` only."""
    q = bf16_to_f64(Q[h][np.asarray(rows)])
    K = np.concatenate([bf16_to_f64(k[h]) for k in K_shards], axis=0)
    V = np.concatenate([bf16_to_f64(v[h]) for v in V_shards], axis=0)
    s = (q @ K.T) / np.sqrt(q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    return (p @ V) / p.sum(axis=1, keepdims=True)
