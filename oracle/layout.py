"""Bit-packed device layout of the Block-GTQ cache (the layout the library writes and reads).

The pages call for a packed-cache serving path (Abstract of "RoPE-Aware Bit
Allocation for KV-Cache Quantization"; Block-GTQ README, backend table) but
print no layout.  The layout fixed for this implementation:

Key codes, per token of one KV head: one bitstream of 2 * sum_j b_j =
128 * avg_k bits = W_K = 4 * avg_k 32-bit words.  Groups follow in width
order 4, 3, 2, 1; code i of the width-w group occupies bits [o_w + w*i,
o_w + w*(i+1)), o_w = bits of the groups before it; bits are LSB-first and a
code may straddle two words.  Device array: u32 [B][Hkv][tile][W_K][64], tile
= t // 64 and lane = t % 64 (word-major inside a tile).

Key norms: fp16 [B][Hkv][tile][64][4]; slot 4 - w holds the width-w group's
norm, absent widths hold 0.

Value codes, per (tile, rotated coordinate i) of one KV head: one bitstream of
64 * b_V bits in which token lane l occupies bits [b_V * l, b_V * (l+1)),
LSB-first = 2 * b_V words.  Device array: u32 [B][Hkv][tile][128][2 * b_V]
(coordinate-major inside a tile).

Value norms: fp16 [B][Hkv][tile][64].

Cache positions at or beyond the sequence length hold zero bits.
"""
from __future__ import annotations

import numpy as np

from .quant import groups_for

TILE = 64
HEAD_DIM = 128


def k_words_per_token(bits_row) -> int:
    total = 2 * int(np.asarray(bits_row, dtype=np.int64).sum())
    if total % 32:
        raise ValueError("key bitstream is not a whole number of words")
    return total // 32


def k_bit_offsets(bits_row) -> tuple[np.ndarray, np.ndarray]:
    """(widths, start bit) of every key code position, in stream order."""
    widths = np.concatenate([np.full(c.size, w, dtype=np.int64) for w, c in groups_for(bits_row)]
                            or [np.zeros(0, np.int64)])
    starts = np.concatenate([[0], np.cumsum(widths)[:-1]]).astype(np.int64) if widths.size else widths
    return widths, starts


def pack_bits(codes: np.ndarray, widths: np.ndarray, n_words: int) -> np.ndarray:
    """Pack codes [M, n] with per-position widths into LSB-first u32 words [M, n_words]."""
    codes = np.asarray(codes, dtype=np.uint64)
    m = codes.shape[0]
    words = np.zeros((m, n_words + 1), dtype=np.uint64)
    off = 0
    for p, w in enumerate(np.asarray(widths, dtype=np.int64)):
        v = codes[:, p] & np.uint64((1 << int(w)) - 1)
        wi, sh = off // 32, off % 32
        v = v << np.uint64(sh)
        words[:, wi] |= v & np.uint64(0xFFFFFFFF)
        words[:, wi + 1] |= v >> np.uint64(32)
        off += int(w)
    if np.any(words[:, n_words]):
        raise ValueError("codes overflow the word count")
    return words[:, :n_words].astype(np.uint32)


def unpack_bits(words: np.ndarray, widths: np.ndarray) -> np.ndarray:
    """Inverse of pack_bits: u32 words [M, n_words] -> codes [M, n] (uint8)."""
    words = np.asarray(words, dtype=np.uint64)
    m = words.shape[0]
    ext = np.concatenate([words, np.zeros((m, 1), np.uint64)], axis=1)
    out = np.zeros((m, len(widths)), dtype=np.uint8)
    off = 0
    for p, w in enumerate(np.asarray(widths, dtype=np.int64)):
        wi, sh = off // 32, off % 32
        pair = ext[:, wi] | (ext[:, wi + 1] << np.uint64(32))
        out[:, p] = ((pair >> np.uint64(sh)) & np.uint64((1 << int(w)) - 1)).astype(np.uint8)
        off += int(w)
    return out


def pack_k(codes: np.ndarray, norm_bits: np.ndarray, bits_row, n_tiles: int):
    """One KV head of one sequence: codes [T, d_nz], norm slots [T, 4] -> (u32 [tiles, W_K, 64], u16 [tiles, 64, 4])."""
    t = codes.shape[0]
    assert t <= n_tiles * TILE
    widths, _ = k_bit_offsets(bits_row)
    wk = k_words_per_token(bits_row)
    tok_words = np.zeros((n_tiles * TILE, wk), dtype=np.uint32)
    tok_words[:t] = pack_bits(codes, widths, wk)
    k_arr = tok_words.reshape(n_tiles, TILE, wk).transpose(0, 2, 1).copy()
    nrm = np.zeros((n_tiles * TILE, 4), dtype=np.uint16)
    nrm[:t] = norm_bits
    return k_arr, nrm.reshape(n_tiles, TILE, 4)


def unpack_k(k_arr: np.ndarray, k_norms: np.ndarray, bits_row, t: int):
    """Inverse of pack_k for the first t tokens."""
    widths, _ = k_bit_offsets(bits_row)
    tok_words = k_arr.transpose(0, 2, 1).reshape(-1, k_arr.shape[1])[:t]
    return unpack_bits(tok_words, widths), k_norms.reshape(-1, 4)[:t]


def pack_v(codes: np.ndarray, norm_bits: np.ndarray, v_bits: int, n_tiles: int):
    """One KV head of one sequence: codes [T, 128], norms [T] -> (u32 [tiles, 128, 2b], u16 [tiles, 64])."""
    t = codes.shape[0]
    full = np.zeros((n_tiles * TILE, HEAD_DIM), dtype=np.uint8)
    full[:t] = codes
    per_coord = full.reshape(n_tiles, TILE, HEAD_DIM).transpose(0, 2, 1).reshape(-1, TILE)
    words = pack_bits(per_coord, np.full(TILE, v_bits), 2 * v_bits)
    nrm = np.zeros(n_tiles * TILE, dtype=np.uint16)
    nrm[:t] = norm_bits
    return words.reshape(n_tiles, HEAD_DIM, 2 * v_bits), nrm.reshape(n_tiles, TILE)


def unpack_v(v_arr: np.ndarray, v_norms: np.ndarray, v_bits: int, t: int):
    n_tiles = v_arr.shape[0]
    per_coord = unpack_bits(v_arr.reshape(-1, 2 * v_bits), np.full(TILE, v_bits))
    codes = per_coord.reshape(n_tiles, HEAD_DIM, TILE).transpose(0, 2, 1).reshape(-1, HEAD_DIM)
    return codes[:t], v_norms.reshape(-1)[:t]
