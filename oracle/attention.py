"""Decode attention over a dequantised cache (the quantize -> dequantize -> SDPA reference path).

Block-GTQ README, backend table paragraph: quality results come from a
reference path that quantises, dequantises and runs plain scaled dot-product
attention; the fused packed-cache kernel is the fast path for the same
computation.  This oracle is that reference path in float64:

  l_t = s * (q . k_hat_t),  p = softmax(l) over t in [0, seq_len)  (max subtracted),
  o = sum_t p_t v_hat_t,

with q the fp16 post-RoPE query taken exactly as float64, s = 1/sqrt(128)
unless given, and o = 0 for seq_len = 0 (reading: an empty cache attends to
nothing).
"""
from __future__ import annotations

import math

import numpy as np


def softmax_attention(q: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, scale: float) -> np.ndarray:
    """o for one query vector q [d] over k_hat, v_hat [T, d] (float64)."""
    t = k_hat.shape[0]
    if t == 0:
        return np.zeros(v_hat.shape[1])
    logits = scale * (k_hat @ q)
    m = logits.max()
    p = np.exp(logits - m)
    return (p @ v_hat) / p.sum()


def decode_attention(q16: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, seq_len: int,
                     scale: float | None = None) -> np.ndarray:
    """One sequence: q16 [Hq, d] fp16, k_hat/v_hat [T, Hkv, d] float64 -> o [Hq, d] float64.

    Query head h reads KV head h // (Hq / Hkv).
    """
    hq, d = q16.shape
    hkv = k_hat.shape[1]
    g = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    out = np.zeros((hq, d))
    for h in range(hq):
        kv = h // g
        out[h] = softmax_attention(q[h], k_hat[:seq_len, kv], v_hat[:seq_len, kv], scale)
    return out
