"""Seeded Haar rotations for the TurboQuant-MSE groups.

The pages name a random rotation inside TurboQuant-MSE but fix neither the
rotation family nor the random stream (Block-GTQ README introduction; the
TurboQuant entry of the "Builds on" list on the mlsanity index page).  The
reading taken: a Haar-distributed orthogonal matrix per (layer, KV head,
tensor, width) drawn from a seeded stream --

* SplitMix64 (Steele, Lea & Flood, OOPSLA 2014): state += 0x9E3779B97F4A7C15,
  output = mix(state) with the published mixer (xor-shift 30, multiply
  0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB, xor-shift 31).
* The stream state starts at 0 and absorbs the fields (seed, layer, kvh,
  tensor, width, d) in that order, each as state <- mix((state ^ field) +
  0x9E3779B97F4A7C15), i.e. one SplitMix64 step taken from state ^ field.
* Uniforms u = (x >> 11) * 2^-53 in [0, 1).
* Box-Muller pairs z0 = r cos(2 pi u2), z1 = r sin(2 pi u2) with r =
  sqrt(-2 ln(1 - u1)), filling a d x d Gaussian matrix row-major, z0 first.
* Orthogonalisation G = Q R and Pi = Q diag(sign R_ii), sign(0) = +1
  (Mezzadri, "How to generate random matrices from the classical compact
  groups", Notices AMS 2007), which is unique, so any QR routine gives the
  same Pi up to rounding.  The QR here is LAPACK's (numpy.linalg.qr).

tensor is 0 for keys and 1 for values.  Encoding computes y = Pi x.
"""
from __future__ import annotations

import math

import numpy as np

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def _mix(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


class SplitMix64:
    """SplitMix64 generator on Python integers."""

    def __init__(self, state: int = 0):
        self.state = state & _M64

    def next(self) -> int:
        self.state = (self.state + _GAMMA) & _M64
        return _mix(self.state)

    def absorb(self, field: int) -> None:
        self.state = _mix(((self.state ^ (field & _M64)) + _GAMMA) & _M64)

    def uniform(self) -> float:
        return (self.next() >> 11) * (1.0 / 9007199254740992.0)


def seeded_stream(seed: int, layer: int, kvh: int, tensor: int, width: int, d: int) -> SplitMix64:
    g = SplitMix64(0)
    for f in (seed, layer, kvh, tensor, width, d):
        g.absorb(f)
    return g


def gaussian_matrix(gen: SplitMix64, d: int) -> np.ndarray:
    """d x d standard Gaussian matrix by Box-Muller, row-major, z0 then z1 (d*d must be even)."""
    out = np.empty(d * d, dtype=np.float64)
    for i in range(0, d * d, 2):
        u1 = gen.uniform()
        u2 = gen.uniform()
        r = math.sqrt(-2.0 * math.log(1.0 - u1))
        out[i] = r * math.cos(2.0 * math.pi * u2)
        out[i + 1] = r * math.sin(2.0 * math.pi * u2)
    return out.reshape(d, d)


def haar_rotation(g: np.ndarray) -> np.ndarray:
    """Pi = Q diag(sign R_ii) from G = QR, with sign(0) = +1."""
    q, r = np.linalg.qr(g)
    s = np.where(np.diag(r) < 0.0, -1.0, 1.0)
    return q * s[None, :]


def rotation_for(seed: int, layer: int, kvh: int, tensor: int, width: int, d: int) -> np.ndarray:
    """The d x d rotation of one (layer, KV head, tensor, width) group."""
    if d <= 0 or d % 2:
        raise ValueError("group size must be positive and even")
    return haar_rotation(gaussian_matrix(seeded_stream(seed, layer, kvh, tensor, width, d), d))
