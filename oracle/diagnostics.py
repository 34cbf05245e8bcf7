"""Per-layer RoPE-logit fidelity of a quantised key cache (a reported diagnostic, not parity).

"RoPE-Aware Bit Allocation for KV-Cache Quantization", Abstract: Block-GTQ is
judged by how well it preserves the RoPE query-key logits, as the per-layer
mean absolute error against the unquantised logits, K-only at 2 and 3 bits per
coordinate, against uniform TQ-MSE at the same budget.  Block-GTQ README,
per-layer diagnostic section: the MAE is taken over a window of the last
M = 1024 positions (``--window-M 1024``).

Reading taken (the pages do not write the formula): for queries q_t and keys
k_s at positions in the window (both post-RoPE, the keys as stored before
quantisation), over every query head h (KV head h // G) and every causal pair
s <= t in the window,

  MAE = mean |q_t,h . k_hat_s,kvh - q_t,h . k_s,kvh|     (unscaled logits)

with k_hat the dequantised key.
"""
from __future__ import annotations

import numpy as np


def logit_mae(q: np.ndarray, k: np.ndarray, k_hat: np.ndarray, group: int) -> float:
    """q [M, Hq, d], k and k_hat [M, Hkv, d] (any float dtype; computed in float64) -> MAE."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    k_hat = np.asarray(k_hat, np.float64)
    m, hq, _ = q.shape
    causal = np.tril(np.ones((m, m), dtype=bool))          # [t, s]: s <= t
    total = 0.0
    for h in range(hq):
        kv = h // group
        err = q[:, h] @ (k_hat[:, kv] - k[:, kv]).T         # [t, s]
        total += np.abs(err[causal]).sum()
    return total / (hq * causal.sum())
