"""Label-free RoPE-block energy and greedy integer bit allocation.

Abstract of "RoPE-Aware Bit Allocation for KV-Cache Quantization": for each
layer and KV head, Block-GTQ scores every RoPE block with a label-free energy
and greedily allocates integer bit widths by marginal gain.  The Block-GTQ
README (introduction and calibration paragraphs) adds that the score is a
Q/K energy computed from saved Q/K activations of one forward pass, and that
bits shift toward high-energy blocks under a fixed average budget.

Readings taken where the pages are silent:

* Energy of block j of KV head h, whose coordinates are (a_j, b_j) =
  (j, j+64) under the half-split pairing or (2j, 2j+1) under the interleaved
  one (oracle.rope.block_pairs):
    E_{h,j} = Eq_{h,j} * Ek_{h,j},
    Eq_{h,j} = sum_{t, h' in grp(h)} (q_{t,h',a_j}^2 + q_{t,h',b_j}^2) / (n_cal * G),
    Ek_{h,j} = sum_t (k_{t,h,a_j}^2 + k_{t,h,b_j}^2) / n_cal,
  with grp(h) = {hG, ..., hG+G-1}.  The logit term of block j is bounded by
  |q_j| |k_j| and RoPE preserves block norms, so this is position-free.
  Each sum is the exact sum of the fp16 squares rounded once to float64;
  then one division and one product, each rounded once.
* Distortion model D(b) = Lloyd-Max MSE of N(0,1) at b bits, D(0) = 1.
* Greedy: start all widths at 0; take avg_bits * n_blocks steps; each step
  adds one bit to the block with the largest gain E_j * (D(b_j) - D(b_j+1))
  among blocks with b_j < 4; ties go to the lowest block index.
"""
from __future__ import annotations

import numpy as np

from .rope import block_pairs


def exact_sum_squares_f16(x16: np.ndarray, axis: int = -1) -> np.ndarray:
    """Exact sum of squares of fp16 values along ``axis``, rounded once to float64.

    Every fp16 value is an integer multiple of 2^-24 below 2^16, so
    k = |x| * 2^24 < 2^40 is an exact integer and x^2 = k^2 * 2^-48.  The sum
    is formed exactly with Python integers and converted with one
    round-to-nearest-even (int -> float conversion is correctly rounded).
    """
    x16 = np.asarray(x16, dtype=np.float16)
    k = (np.abs(x16.astype(np.float64)) * 16777216.0).astype(np.int64)
    kh = k >> 20
    kl = k & ((1 << 20) - 1)
    a = (kh * kh).sum(axis=axis)                 # < 2^40 per term
    b = (2 * kh * kl).sum(axis=axis)
    c = (kl * kl).sum(axis=axis)
    tot = (a.astype(object) << 40) + (b.astype(object) << 20) + c.astype(object)
    return np.asarray(tot, dtype=object).astype(np.float64) * (2.0 ** -48)


def energy(q_cal: np.ndarray, k_cal: np.ndarray, n_kv_heads: int, pairing: str = "half") -> np.ndarray:
    """Block energies E [Hkv, head_dim/2] (float64) from fp16 calibration Q [n, Hq, d] and K [n, Hkv, d]."""
    q_cal = np.asarray(q_cal, dtype=np.float16)
    k_cal = np.asarray(k_cal, dtype=np.float16)
    n, hq, d = q_cal.shape
    assert k_cal.shape == (n, n_kv_heads, d) and d % 2 == 0 and hq % n_kv_heads == 0
    g = hq // n_kv_heads
    nb = d // 2
    a, b = block_pairs(d, pairing)
    out = np.empty((n_kv_heads, nb), dtype=np.float64)
    for h in range(n_kv_heads):
        qh = q_cal[:, h * g:(h + 1) * g, :]                          # [n, G, d]
        q_pairs = np.concatenate([qh[..., a], qh[..., b]], axis=1)    # [n, 2G, nb]
        k_pairs = np.stack([k_cal[:, h, a], k_cal[:, h, b]], axis=1)  # [n, 2, nb]
        sq = exact_sum_squares_f16(q_pairs.transpose(2, 0, 1).reshape(nb, -1))
        sk = exact_sum_squares_f16(k_pairs.transpose(2, 0, 1).reshape(nb, -1))
        eq = sq / float(n * g)
        ek = sk / float(n)
        out[h] = eq * ek
    return out


def greedy_allocate(e_row: np.ndarray, avg_bits: int, dist: np.ndarray, max_bits: int = 4) -> np.ndarray:
    """Integer widths (int8, one per block) for one KV head.

    ``dist`` is D(0..max_bits); the gain of raising block j from b to b+1 is
    e_row[j] * (D(b) - D(b+1)).  Budget: sum_j b_j = avg_bits * n_blocks.
    """
    nb = len(e_row)
    if not 0 <= avg_bits <= max_bits:
        raise ValueError("avg_bits out of range")
    dd = [float(dist[b]) - float(dist[b + 1]) for b in range(max_bits)]
    bits = [0] * nb
    e = [float(v) for v in e_row]
    for _ in range(avg_bits * nb):
        best, best_gain = -1, 0.0
        for j in range(nb):
            if bits[j] < max_bits:
                gain = e[j] * dd[bits[j]]
                if best < 0 or gain > best_gain:
                    best, best_gain = j, gain
        bits[best] += 1
    return np.array(bits, dtype=np.int8)
