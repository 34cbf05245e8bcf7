"""RoPE and its 2-D frequency-block decomposition of a logit.

Abstract of "RoPE-Aware Bit Allocation for KV-Cache Quantization" and the
Block-GTQ README introduction: under RoPE a cached key's contribution to a
future logit is a position-dependent sum over two-dimensional frequency
blocks.  The pages name no pairing of coordinates into blocks, so both
conventions in use are supported:

* "half" (the default, rotate-half): block j = coordinates (j, j + d/2);
* "interleaved": block j = coordinates (2j, 2j + 1), the pair read as the
  complex number x[2j] + i x[2j+1].

Either way block j has frequency omega_j = theta^(-2j/d) and at position p its
pair is rotated by the angle p * omega_j.  Then
q'(m) . k'(n) = sum_j q_j^T R(omega_j (n - m)) k_j for a query at position m
and a key at position n, which block_logits returns term by term.
"""
from __future__ import annotations

import numpy as np

PAIRINGS = ("half", "interleaved")


def block_pairs(d: int, pairing: str = "half") -> tuple[np.ndarray, np.ndarray]:
    """(first, second) coordinate of every 2-D block j = 0 .. d/2 - 1."""
    j = np.arange(d // 2)
    if pairing == "half":
        return j, j + d // 2
    if pairing == "interleaved":
        return 2 * j, 2 * j + 1
    raise ValueError("pairing must be 'half' or 'interleaved'")


def _omega(d: int, theta: float) -> np.ndarray:
    return theta ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)


def rope_blocks(x: np.ndarray, pos: float, theta: float, pairing: str = "half") -> np.ndarray:
    """Rotate one float64 vector x [d] to position ``pos``."""
    d = x.shape[-1]
    a, b = block_pairs(d, pairing)
    ang = pos * _omega(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x, dtype=np.float64)
    out[a] = x[a] * c - x[b] * s
    out[b] = x[a] * s + x[b] * c
    return out


def block_logits(q: np.ndarray, k: np.ndarray, m: float, n: float, theta: float,
                 pairing: str = "half") -> np.ndarray:
    """Per-block terms q_j^T R(omega_j (n - m)) k_j for pre-RoPE q (at m) and k (at n)."""
    d = q.shape[-1]
    a, b = block_pairs(d, pairing)
    ang = (n - m) * _omega(d, theta)
    c, s = np.cos(ang), np.sin(ang)
    k_rot0 = k[a] * c - k[b] * s
    k_rot1 = k[a] * s + k[b] * c
    return q[a] * k_rot0 + q[b] * k_rot1
