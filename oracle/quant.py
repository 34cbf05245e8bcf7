"""TurboQuant-MSE group encoder and decoder (keys with Block-GTQ widths, values uniform).

Abstract of "RoPE-Aware Bit Allocation for KV-Cache Quantization": Block-GTQ
is a bit allocator built on TurboQuant-MSE; K/V budgets are written KxVy
(K2V2, K3V2, K3V3) and values are quantised at a uniform width.  The pages
do not spell out the encoder; the readings taken are:

* Groups (keys): one group per width w present in the allocation, in the
  order w = 4, 3, 2, 1.  Group w holds the blocks j with b_j = w in
  ascending j, each block contributing its two coordinates next to each
  other: (j, j+64) under the half-split RoPE pairing, (2j, 2j+1) under the
  interleaved one.  Zero-width blocks are not stored and decode to 0.
* Values: one group of all 128 coordinates in natural order at width b_V.
* Per token and group: n = ||x_g|| in float64 (exact sum of the fp16 squares
  rounded once, then a correctly rounded sqrt); y = Pi x_g / n (y = 0 when
  n = 0); z = sqrt(d_g) * y; code_i = #{t_k < z_i} with the N(0,1) Lloyd-Max
  thresholds of the group width (a tie goes to the lower code); the stored
  norm is fp16(n) with a single round-to-nearest-even from float64.
* Decode: x_hat_g = fp16(n) * Pi^T (c[code] / sqrt(d_g)), no renormalisation.
"""
from __future__ import annotations

import math

import numpy as np

from .alloc import exact_sum_squares_f16
from .codebook import lloyd_max
from .rope import block_pairs
from .rotation import rotation_for

HEAD_DIM = 128
N_BLOCKS = 64
K_TENSOR, V_TENSOR = 0, 1


def f16_bits(x) -> np.ndarray:
    """IEEE binary16 bit patterns of float64 values, one round-to-nearest-even step."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_value(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def groups_for(bits_row, pairing: str = "half") -> list[tuple[int, np.ndarray]]:
    """[(width, coordinate indices)] for widths 4, 3, 2, 1 that are present."""
    bits_row = np.asarray(bits_row)
    first, second = block_pairs(HEAD_DIM, pairing)
    out = []
    for w in (4, 3, 2, 1):
        blocks = np.nonzero(bits_row == w)[0]
        if blocks.size:
            coords = np.stack([first[blocks], second[blocks]], axis=1).reshape(-1)
            out.append((w, coords))
    return out


def encode_groups(x16: np.ndarray, groups, rotations, sum_sq=None):
    """Encode fp16 rows x16 [N, 128] group by group.

    ``groups`` is [(w, coords)], ``rotations`` the matching list of Pi.
    Returns (codes [N, sum d_g] uint8 in group order, norms [N, n_groups] float64).
    """
    x16 = np.asarray(x16, dtype=np.float16)
    n_rows = x16.shape[0]
    codes, norms = [], []
    for (w, coords), pi in zip(groups, rotations):
        xg16 = x16[:, coords]
        d = coords.size
        ss = exact_sum_squares_f16(xg16, axis=1)
        n = np.sqrt(ss)
        xg = xg16.astype(np.float64)
        py = xg @ pi.T
        safe = np.where(n > 0.0, n, 1.0)
        y = np.where((n > 0.0)[:, None], py / safe[:, None], 0.0)
        z = math.sqrt(d) * y
        thr = lloyd_max(w)[1]
        codes.append(np.searchsorted(thr, z, side="left").astype(np.uint8))
        norms.append(n)
    if not codes:
        return np.zeros((n_rows, 0), np.uint8), np.zeros((n_rows, 0))
    return np.concatenate(codes, axis=1), np.stack(norms, axis=1)


def k_rotations(bits_row, seed: int, layer: int, kvh: int):
    return [rotation_for(seed, layer, kvh, K_TENSOR, w, c.size) for w, c in groups_for(bits_row)]


def v_rotation(v_bits: int, seed: int, layer: int, kvh: int):
    return rotation_for(seed, layer, kvh, V_TENSOR, v_bits, HEAD_DIM)


def encode_k(k16: np.ndarray, bits_row, seed: int, layer: int, kvh: int, rots=None, pairing: str = "half"):
    """Keys of one KV head, fp16 [N, 128] -> (codes [N, d_nz] uint8, norm bits [N, 4] uint16).

    Norm slot 4 - w holds the fp16 norm of the width-w group; absent slots are 0.
    """
    groups = groups_for(bits_row, pairing)
    if rots is None:
        rots = k_rotations(bits_row, seed, layer, kvh)
    codes, norms = encode_groups(k16, groups, rots)
    slots = np.zeros((k16.shape[0], 4), dtype=np.uint16)
    for gi, (w, _) in enumerate(groups):
        slots[:, 4 - w] = f16_bits(norms[:, gi])
    return codes, slots


def encode_v(v16: np.ndarray, v_bits: int, seed: int, layer: int, kvh: int, rot=None):
    """Values of one KV head, fp16 [N, 128] -> (codes [N, 128] uint8, norm bits [N] uint16)."""
    coords = np.arange(HEAD_DIM)
    if rot is None:
        rot = v_rotation(v_bits, seed, layer, kvh)
    codes, norms = encode_groups(v16, [(v_bits, coords)], [rot])
    return codes, f16_bits(norms[:, 0])


def dequant_k(codes, norm_bits, bits_row, seed: int, layer: int, kvh: int, rots=None,
              pairing: str = "half") -> np.ndarray:
    """Reconstructed keys [N, 128] float64 from codes [N, d_nz] and norm slots [N, 4]."""
    groups = groups_for(bits_row, pairing)
    if rots is None:
        rots = k_rotations(bits_row, seed, layer, kvh)
    n_rows = codes.shape[0]
    out = np.zeros((n_rows, HEAD_DIM), dtype=np.float64)
    off = 0
    for (w, coords), pi in zip(groups, rots):
        d = coords.size
        cent = lloyd_max(w)[0]
        yhat = cent[codes[:, off:off + d].astype(np.int64)] / math.sqrt(d)
        nrm = f16_value(norm_bits[:, 4 - w])
        out[:, coords] = nrm[:, None] * (yhat @ pi)
        off += d
    return out


def dequant_v(codes, norm_bits, v_bits: int, seed: int, layer: int, kvh: int, rot=None) -> np.ndarray:
    if rot is None:
        rot = v_rotation(v_bits, seed, layer, kvh)
    cent = lloyd_max(v_bits)[0]
    yhat = cent[codes.astype(np.int64)] / math.sqrt(HEAD_DIM)
    return f16_value(norm_bits)[:, None] * (yhat @ rot)
