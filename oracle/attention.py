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


def buffered_positions(seq_len: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Boolean mask [seq_len]: True where a token is kept in fp16 (the first ``n_sink`` tokens and the
    last ``n_recent``), False where the packed cache serves it."""
    t = np.arange(seq_len)
    return (t < n_sink) | (t >= seq_len - n_recent)


def decode_attention_buffered(q16: np.ndarray, k16: np.ndarray, v16: np.ndarray, k_hat: np.ndarray,
                              v_hat: np.ndarray, seq_len: int, n_sink: int, n_recent: int,
                              scale: float | None = None) -> np.ndarray:
    """Decode attention with an fp16 sink and recent window (the Block-GTQ README's "withbuffer"
    setting of its AIME runs: 4 attention-sink tokens and a 128-token recent window in fp16).

    Reading: token t of a sequence of length T attends with its original fp16 key and value
    (taken exactly as float64) when t < n_sink or t >= T - n_recent, and with the dequantised
    k_hat_t, v_hat_t otherwise; the softmax and the weighted sum are those of decode_attention.
    q16 [Hq, d]; k16, v16 fp16 and k_hat, v_hat float64, all [T', Hkv, d] with T' >= seq_len.
    """
    keep = buffered_positions(seq_len, n_sink, n_recent)[:, None, None]
    k = np.where(keep, np.asarray(k16[:seq_len], np.float16).astype(np.float64), k_hat[:seq_len])
    v = np.where(keep, np.asarray(v16[:seq_len], np.float16).astype(np.float64), v_hat[:seq_len])
    return decode_attention(q16, k, v, seq_len, scale)
