"""GPU parity of the fp16 decode-attention baseline (bgtq_fp16_decode_attn) against the
oracle's plain softmax attention on the same fp16 keys and values taken exactly as float64.
Tolerance: 2e-3 relative L2 per (sequence, query head), as for the packed path (fp16 I/O,
fp32 accumulation)."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from gpu_case import log, rel_l2, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module")
def bg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_bgtq_amd as m
    m.load()
    return m


def _run(bg, q, k, v, seq_lens, max_seq_len, scale=None):
    import torch
    b, hq, _ = q.shape
    _, cap, hkv, _ = k.shape
    out = torch.empty((b, hq, 128), dtype=torch.int16, device="cuda")
    ws = torch.empty(bg.fp16_workspace_size(b, hkv, hq, max_seq_len), dtype=torch.uint8, device="cuda")
    sl = torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    torch.cuda.synchronize()
    log("fp16 decode: batch %d, %d/%d heads, capacity %d, max_seq_len %d" % (b, hq, hkv, cap, max_seq_len))
    bg.fp16_decode_attn(qd, kd, vd, sl, max_seq_len, out, ws, softmax_scale=scale)
    torch.cuda.synchronize()
    log("fp16 decode done")
    return out.cpu().numpy().view(np.float16).astype(np.float64)


def _check(got, q, k, v, seq_lens, scale=None):
    b, hq, _ = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    s = scale if scale is not None else 1 / math.sqrt(128)
    worst = 0.0
    for i in range(b):
        for h in range(hq):
            if seq_lens[i] == 0:
                assert np.all(got[i, h] == 0.0)
                continue
            t = seq_lens[i]
            ref = oracle.softmax_attention(q[i, h].astype(np.float64), k[i, :t, h // g].astype(np.float64),
                                           v[i, :t, h // g].astype(np.float64), s)
            r = rel_l2(got[i, h], ref)
            worst = max(worst, float(r))
            assert r <= TOL, (i, h, r)
    log("fp16 decode worst rel-L2 %.3e" % worst)


def _inputs(cid, batch, t, cap, hkv=None, hq=None):
    log("inputs: config %d, batch %d, T %d, capacity %d" % (cid, batch, t, cap))
    cfg = synth.small(cid, seq_len=t, batch=batch)
    if hkv is not None:
        cfg = synth.small(cid, seq_len=t, batch=batch, n_kv_heads=hkv, n_q_heads=hq)
    k = np.zeros((batch, cap, cfg.n_kv_heads, 128), np.float16)
    v = np.zeros_like(k)
    for s in range(batch):
        k[s, :t] = synth.keys(cfg, seq=s, count=t)
        v[s, :t] = synth.values(cfg, seq=s, count=t)
    q = np.stack([synth.query(cfg, seq=s) for s in range(batch)])
    return q, k, v


@pytest.mark.parametrize("cid,t", [(1, 4096), (1, 1), (1, 100), (2, 2000), (3, 3000), (5, 1500)])
def test_fp16_decode_matches_oracle(bg, cid, t):
    q, k, v = _inputs(cid, 1, t, t + 37)
    got = _run(bg, q, k, v, [t], t)
    _check(got, q, k, v, [t])


@pytest.mark.parametrize("g", [1, 2, 4, 8])
def test_fp16_decode_group_sizes(bg, g):
    q, k, v = _inputs(2, 1, 777, 800, hkv=2, hq=2 * g)
    got = _run(bg, q, k, v, [777], 777)
    _check(got, q, k, v, [777])


def test_fp16_decode_ragged_batch_and_empty(bg):
    lens = [0, 1, 64, 700, 1100]
    q, k, v = _inputs(4, 5, 1100, 1152)
    got = _run(bg, q, k, v, lens, 1100)
    _check(got, q, k, v, lens)


def test_fp16_decode_custom_scale(bg):
    q, k, v = _inputs(1, 1, 500, 512)
    got = _run(bg, q, k, v, [500], 500, scale=0.05)
    _check(got, q, k, v, [500], scale=0.05)


def test_fp16_decode_full_size_128k_sampled_heads(bg):
    """The 128K Llama-3.1-8B-shaped layer at full length in the benchmark's launch shape; the
    query heads of KV heads 0 and 5 against the oracle."""
    cfg = synth.CONFIGS[3]
    t = cfg.seq_len
    k = synth.keys(cfg, count=t)[None]
    v = synth.values(cfg, count=t)[None]
    q = synth.query(cfg)[None]
    got = _run(bg, q, k, v, [t], t)
    for kvh in (0, 5):
        for h in range(kvh * cfg.group, (kvh + 1) * cfg.group):
            ref = oracle.softmax_attention(q[0, h].astype(np.float64), k[0, :, kvh].astype(np.float64),
                                           v[0, :, kvh].astype(np.float64), 1 / math.sqrt(128))
            r = rel_l2(got[0, h], ref)
            log("128K fp16 head %d rel-L2 %.3e" % (h, r))
            assert r <= TOL
