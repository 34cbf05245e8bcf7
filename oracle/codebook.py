"""Lloyd-Max scalar codebooks for a unit Gaussian, in float64.

TurboQuant-MSE (the base encoder named in the Abstract of "RoPE-Aware Bit
Allocation for KV-Cache Quantization" and in the Block-GTQ README
introduction) quantises each coordinate of a randomly rotated unit vector
with a scalar MSE-optimal quantiser for its coordinate distribution.  The
pages do not print the quantiser; the reading taken here is the b-bit
Lloyd-Max quantiser of N(0, 1), computed in float64, applied to
sqrt(d_g) * y so that a group of d_g coordinates uses N(0, 1/d_g).

Procedure (Lloyd 1957 / Max 1960):
  thresholds t_k = (c_{k-1} + c_k) / 2,
  centroids  c_k = (phi(t_k) - phi(t_{k+1})) / (Phi(t_{k+1}) - Phi(t_k)),
iterated from a sorted start until the largest centroid move is <= 1e-15
or 100000 iterations, then made exactly odd-symmetric, c_k <- (c_k -
c_{L-1-k}) / 2, which makes the middle threshold exactly +0.0.

Distortion D(b) = 1 - sum_k p_k c_k^2 (the MSE at the centroid condition),
D(0) = 1 (every coordinate reconstructed as 0).
"""
from __future__ import annotations

import functools
import math

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _pdf(x: float) -> float:
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def _mass(a: float, b: float) -> float:
    """P(a <= X < b) for X ~ N(0,1), using the upper tail when both ends are positive."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / _SQRT2) - math.erfc(b / _SQRT2))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / _SQRT2) - math.erfc(-a / _SQRT2))
    return 1.0 - 0.5 * math.erfc(-a / _SQRT2) - 0.5 * math.erfc(b / _SQRT2)


@functools.lru_cache(maxsize=None)
def lloyd_max(bits: int, tol: float = 1e-15, max_iter: int = 100000):
    """b-bit Lloyd-Max quantiser of N(0,1).

    Returns (centroids [2^b], thresholds [2^b - 1], distortion D(b), iterations).
    Thresholds are the interior cell boundaries; a value z gets code
    #{k : t_k < z}.
    """
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    n = 1 << bits
    # sorted start: evenly spaced over [-2, 2]
    c = [(-2.0 + 4.0 * (k + 0.5) / n) for k in range(n)]
    it = 0
    for it in range(1, max_iter + 1):
        t = [-math.inf] + [0.5 * (c[k - 1] + c[k]) for k in range(1, n)] + [math.inf]
        new = [(_pdf(t[k]) - _pdf(t[k + 1])) / _mass(t[k], t[k + 1]) for k in range(n)]
        move = max(abs(a - b) for a, b in zip(new, c))
        c = new
        if move <= tol:
            break
    c = [(c[k] - c[n - 1 - k]) / 2.0 for k in range(n)]
    t = [0.5 * (c[k - 1] + c[k]) for k in range(1, n)]
    edges = [-math.inf] + t + [math.inf]
    p = [_mass(edges[k], edges[k + 1]) for k in range(n)]
    d = 1.0 - math.fsum(pk * ck * ck for pk, ck in zip(p, c))
    return np.array(c), np.array(t), d, it


def codebooks():
    """{b: (centroids, thresholds)} for b = 1..4."""
    return {b: lloyd_max(b)[:2] for b in range(1, 5)}


def distortion_table() -> np.ndarray:
    """D(b) for b = 0..4 with D(0) = 1."""
    return np.array([1.0] + [lloyd_max(b)[2] for b in range(1, 5)])
