"""Seeded synthetic inputs for the Block-GTQ packed-KV path.

This module only draws inputs. It holds none of the method's arithmetic
(no energy, allocation, codebook, rotation, quantiser or attention); the
oracle and the HIP library both consume what it returns.

Shapes and distributions follow the five workloads of the packed-cache path
(post-RoPE fp16 keys, queries and calibration activations, fp16 values):

* RoPE pairs the coordinates of a 128-wide head into 2-D blocks either
  half-split ("rotate-half", the default: block j is the pair (j, j+64)) or
  interleaved (block j is (2j, 2j+1)), as ``Config.pairing`` says; block j
  is rotated at position p by the angle p * theta**(-2j/128).  RoPE is applied in float64 and the result
  is rounded to fp16 (round-to-nearest-even) in one step.
* Pre-RoPE keys (and queries, drawn the same way from the KV head they
  share) have both coordinates of block j ~ N(0, s_{h,j}^2); values are
  iid N(0, 1).  An interleaved config draws exactly the numbers of its
  half-split twin, with coordinate (j, j+64) of every key, query and
  calibration row moved to (2j, 2j+1).
* Random streams are ``numpy.random.Generator(PCG64(SeedSequence(seed,
  spawn_key=(config, stream, seq))))`` with one stream per tensor kind.
"""
from __future__ import annotations

import dataclasses
import numpy as np

HEAD_DIM = 128
N_BLOCKS = HEAD_DIM // 2

# stream ids inside one config
_S_SCALES, _S_K, _S_V, _S_Q, _S_QCAL, _S_KCAL, _S_OUTLIER, _S_QWIN = 0, 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload (a single attention layer)."""

    cid: int
    name: str
    batch: int
    seq_len: int
    n_kv_heads: int
    n_q_heads: int
    theta: float
    scale_kind: str          # "exp12" (s_j = exp(-j/12)) or "lognormal"
    sigma: float             # log-normal sigma of the per-block energy s^2
    n_outliers: int          # outlier blocks per KV head (std x 8)
    k_bits: int              # average K bits per coordinate
    v_bits: int              # uniform V bits per coordinate
    n_cal: int               # calibration tokens
    append: int = 0          # tokens appended after the prefill cache
    seed: int = 0
    pairing: str = "half"    # RoPE block pairing: "half" (j, j+64) or "interleaved" (2j, 2j+1)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = {
    1: Config(1, "tiny-1head-4k", 1, 4096, 1, 1, 1e4, "exp12", 0.0, 3, 3, 3, 256),
    2: Config(2, "qwen2.5-3b-layer-32k", 1, 32768, 2, 16, 1e6, "lognormal", 1.5, 0, 3, 3, 2048),
    3: Config(3, "llama3.1-8b-layer-128k", 1, 131072, 8, 32, 5e5, "lognormal", 2.0, 4, 2, 2, 2048),
    4: Config(4, "llama3.1-8b-layer-16x32k", 16, 32768, 8, 32, 5e5, "lognormal", 1.5, 0, 3, 2, 2048),
    5: Config(5, "qwen2.5-3b-layer-512k", 1, 524288, 2, 16, 1e6, "exp12", 0.0, 3, 3, 3, 2048,
              append=4096),
}


def _rng(cfg: Config, stream: int, seq: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(cfg.seed, spawn_key=(cfg.cid, stream, seq))
    return np.random.Generator(np.random.PCG64(ss))


def block_scales(cfg: Config) -> np.ndarray:
    """Per-(KV head, block) standard deviation s_{h,j}, float64 [Hkv, 64]."""
    h = cfg.n_kv_heads
    j = np.arange(N_BLOCKS, dtype=np.float64)
    if cfg.scale_kind == "exp12":
        s = np.tile(np.exp(-j / 12.0), (h, 1))
    elif cfg.scale_kind == "lognormal":
        z = _rng(cfg, _S_SCALES).standard_normal((h, N_BLOCKS))
        s = np.sqrt(np.exp(cfg.sigma * z))
    else:
        raise ValueError(cfg.scale_kind)
    if cfg.n_outliers:
        r = _rng(cfg, _S_OUTLIER)
        for hh in range(h):
            idx = r.choice(N_BLOCKS, size=cfg.n_outliers, replace=False)
            s[hh, idx] *= 8.0
    return s


def to_pairing(x: np.ndarray, pairing: str) -> np.ndarray:
    """Move half-split coordinates (j, j+64) of ``x[..., 128]`` to the slots of ``pairing``."""
    if pairing == "half":
        return x
    if pairing != "interleaved":
        raise ValueError("pairing must be 'half' or 'interleaved'")
    out = np.empty_like(x)
    out[..., 0::2] = x[..., :N_BLOCKS]
    out[..., 1::2] = x[..., N_BLOCKS:]
    return out


def rope_f64(x: np.ndarray, pos: np.ndarray, theta: float, pairing: str = "half") -> np.ndarray:
    """RoPE on float64 ``x[..., tokens, heads, 128]`` at positions ``pos``.

    ``pos`` has one entry per token (axis -3 of ``x``).
    """
    if pairing == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
    elif pairing == "half":
        a, b = x[..., :N_BLOCKS], x[..., N_BLOCKS:]
    else:
        raise ValueError("pairing must be 'half' or 'interleaved'")
    j = np.arange(N_BLOCKS, dtype=np.float64)
    omega = theta ** (-2.0 * j / HEAD_DIM)
    ang = pos.astype(np.float64)[:, None] * omega[None, :]          # [T, 64]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    ra, rb = a * c - b * s, a * s + b * c
    out = np.empty_like(x)
    if pairing == "interleaved":
        out[..., 0::2], out[..., 1::2] = ra, rb
    else:
        out[..., :N_BLOCKS], out[..., N_BLOCKS:] = ra, rb
    return out


def _draw_blocks(rng: np.random.Generator, n: int, heads_scale: np.ndarray) -> np.ndarray:
    """float64 [n, H, 128]: block j of head h (coords j and j+64) ~ N(0, s[h,j]^2)."""
    h = heads_scale.shape[0]
    z = rng.standard_normal((n, h, HEAD_DIM))
    s = np.concatenate([heads_scale, heads_scale], axis=1)          # [H, 128]
    return z * s[None, :, :]


def keys(cfg: Config, seq: int = 0, start: int = 0, count: int | None = None,
         chunk: int = 65536) -> np.ndarray:
    """Post-RoPE fp16 keys [count, Hkv, 128] for sequence ``seq``, positions start..start+count-1.

    The draw is chunked so any window is a slice of one fixed full-length draw.
    """
    return _token_tensor(cfg, _S_K, seq, start, count, chunk, rope=True)


def values(cfg: Config, seq: int = 0, start: int = 0, count: int | None = None,
           chunk: int = 65536) -> np.ndarray:
    """fp16 values [count, Hkv, 128], iid N(0, 1)."""
    return _token_tensor(cfg, _S_V, seq, start, count, chunk, rope=False)


def _token_tensor(cfg, stream, seq, start, count, chunk, rope):
    total = cfg.seq_len + cfg.append
    if count is None:
        count = total - start
    assert 0 <= start and start + count <= total
    scales = block_scales(cfg) if rope else np.ones((cfg.n_kv_heads, N_BLOCKS))
    out = np.empty((count, cfg.n_kv_heads, HEAD_DIM), dtype=np.float16)
    # fixed chunk grid of the full-length draw: chunk c covers [c*chunk, (c+1)*chunk)
    c0 = start // chunk
    c1 = (start + count - 1) // chunk if count else c0 - 1
    for c in range(c0, c1 + 1):
        lo, hi = c * chunk, min((c + 1) * chunk, total)
        rng = _rng(cfg, stream, seq * 4096 + c)
        x = _draw_blocks(rng, hi - lo, scales)
        if rope:
            x = rope_f64(to_pairing(x, cfg.pairing), np.arange(lo, hi), cfg.theta, cfg.pairing)
        a, b = max(lo, start), min(hi, start + count)
        out[a - start:b - start] = x[a - lo:b - lo].astype(np.float16)
    return out


def query(cfg: Config, seq: int = 0, pos: int | None = None) -> np.ndarray:
    """One post-RoPE fp16 decode query per sequence: [Hq, 128] at position ``pos`` (default T)."""
    if pos is None:
        pos = cfg.seq_len
    rng = _rng(cfg, _S_Q, seq)
    sc = np.repeat(block_scales(cfg), cfg.group, axis=0)             # [Hq, 64]
    x = to_pairing(_draw_blocks(rng, 1, sc), cfg.pairing)
    return rope_f64(x, np.array([pos]), cfg.theta, cfg.pairing)[0].astype(np.float16)


def queries(cfg: Config, seq: int = 0, start: int = 0, count: int = 1) -> np.ndarray:
    """Post-RoPE fp16 queries [count, Hq, 128] at positions start..start+count-1, one independent
    draw per position (drawn like the keys of their KV head), for windowed logit diagnostics."""
    rng = _rng(cfg, _S_QWIN, seq)
    sc = np.repeat(block_scales(cfg), cfg.group, axis=0)             # [Hq, 64]
    x = to_pairing(_draw_blocks(rng, count, sc), cfg.pairing)
    return rope_f64(x, np.arange(start, start + count), cfg.theta, cfg.pairing).astype(np.float16)


def calibration(cfg: Config) -> tuple[np.ndarray, np.ndarray]:
    """Calibration activations (post-RoPE fp16) at positions 0..n_cal-1.

    Returns (q_cal [n_cal, Hq, 128], k_cal [n_cal, Hkv, 128]).
    """
    n = cfg.n_cal
    sk = block_scales(cfg)
    sq = np.repeat(sk, cfg.group, axis=0)
    pos = np.arange(n)
    q = rope_f64(to_pairing(_draw_blocks(_rng(cfg, _S_QCAL), n, sq), cfg.pairing), pos, cfg.theta, cfg.pairing)
    k = rope_f64(to_pairing(_draw_blocks(_rng(cfg, _S_KCAL), n, sk), cfg.pairing), pos, cfg.theta, cfg.pairing)
    return q.astype(np.float16), k.astype(np.float16)


def small(cfg_id: int, seq_len: int | None = None, batch: int | None = None,
          n_cal: int | None = None, **kw) -> Config:
    """A reduced copy of a config (same distributions, smaller sizes) for quick parity cases."""
    c = CONFIGS[cfg_id]
    rep = {}
    if seq_len is not None:
        rep["seq_len"] = seq_len
    if batch is not None:
        rep["batch"] = batch
    if n_cal is not None:
        rep["n_cal"] = n_cal
    rep.update(kw)
    return dataclasses.replace(c, **rep)


__all__ = ["Config", "CONFIGS", "HEAD_DIM", "N_BLOCKS", "block_scales", "rope_f64", "to_pairing", "keys",
           "values", "query", "queries", "calibration", "small"]
