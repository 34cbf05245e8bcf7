"""RoPE and its 2-D frequency-block decomposition of a logit.

Abstract of "RoPE-Aware Bit Allocation for KV-Cache Quantization" and the
Block-GTQ README introduction: under RoPE a cached key's contribution to a
future logit is a position-dependent sum over two-dimensional frequency
blocks.  Reading taken for the pairing (the pages name none): the half-split
convention, block j = coordinates (j, j + d/2) with frequency
omega_j = theta^(-2j/d); at position p the pair is rotated by p * omega_j.

Then q'(m) . k'(n) = sum_j q_j^T R(omega_j (n - m)) k_j for a query at
position m and a key at position n, which block_logits returns term by term.
"""
from __future__ import annotations

import numpy as np


def _omega(d: int, theta: float) -> np.ndarray:
    return theta ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)


def rope_blocks(x: np.ndarray, pos: float, theta: float) -> np.ndarray:
    """Rotate one float64 vector x [d] to position ``pos``."""
    d = x.shape[-1]
    h = d // 2
    ang = pos * _omega(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x, dtype=np.float64)
    out[:h] = x[:h] * c - x[h:] * s
    out[h:] = x[:h] * s + x[h:] * c
    return out


def block_logits(q: np.ndarray, k: np.ndarray, m: float, n: float, theta: float) -> np.ndarray:
    """Per-block terms q_j^T R(omega_j (n - m)) k_j for pre-RoPE q (at m) and k (at n)."""
    d = q.shape[-1]
    h = d // 2
    a = (n - m) * _omega(d, theta)
    c, s = np.cos(a), np.sin(a)
    k_rot0 = k[:h] * c - k[h:] * s
    k_rot1 = k[:h] * s + k[h:] * c
    return q[:h] * k_rot0 + q[h:] * k_rot1
