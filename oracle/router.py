"""Top-k router oracle, plain numpy in fp64.

TEST INFRASTRUCTURE, NOT THE PRODUCT: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this. It shares nothing with the HIP path.

What is computed (pages: "The Pivot to Real Hardware...", Input Knowledge Required, item 1 on the
MoE architecture, and "The Weight-Streaming Threshold...", Input Knowledge Required, on the gating
network that picks each token's experts; the softmax / top-k / renormalise recipe is the one the
workload configurations state for the routing): for each token m with router logits l[m, 0..E),

  ids[m]  = the k experts with the largest logits, largest first; among equal logits the lower
            expert index comes first (a plain stable order);
  w[m, j] = exp(l[m, ids[m, j]]) / sum_i exp(l[m, ids[m, i]])   (fp64),

which equals a softmax over all E logits renormalised over the chosen k, since the softmax's common
normaliser cancels. Logits are fp32 and compared as such, so the selection is exact; the weights are
fp64 with no intermediate rounding. Logits may be -inf (a masked expert) as long as each token has a
finite largest logit; NaN logits are outside the domain and rejected.
"""
from __future__ import annotations

import numpy as np

__all__ = ["route"]


def route(logits, k: int):
    """logits float32 [M, E] -> (ids int32 [M, k], weights float64 [M, k])."""
    logits = np.asarray(logits, dtype=np.float32)
    if logits.ndim != 2:
        raise ValueError("logits must be [M, E]")
    M, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError(f"k = {k} outside [1, E = {E}]")
    if np.isnan(logits).any():
        raise ValueError("NaN logits are outside the router's domain")
    ids = np.empty((M, k), dtype=np.int32)
    w = np.empty((M, k), dtype=np.float64)
    for m in range(M):
        row = [float(v) for v in logits[m]]          # exact: fp32 values widened to Python floats
        order = sorted(range(E), key=lambda e: (-row[e], e))
        chosen = order[:k]
        top = row[chosen[0]]
        if not np.isfinite(top):
            raise ValueError(f"token {m}: no finite logit")
        z = [np.exp(row[e] - top) for e in chosen]    # fp64; masked (-inf) experts give 0
        s = sum(z)
        ids[m] = chosen
        w[m] = [v / s for v in z]
    return ids, w
