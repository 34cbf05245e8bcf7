"""K-only key logits from the packed cache (bgtq_key_logits) against the oracle, and the per-layer
RoPE-logit MAE taken from the library's output ("RoPE-Aware Bit Allocation for KV-Cache
Quantization", Abstract: K-only at 2 and 3 bits per coordinate; README per-layer diagnostic).
Expected values come from the oracle's encode and dequantisation only."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from gpu_case import OracleHead, log, ref_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bg():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_bgtq_amd as m
    m.load()
    return m


def _library_logits(bg, plan, cache, q16, t0, n_k):
    """q16 [batch, n_q, Hq, 128] fp16 -> logits [batch, Hq, n_q, n_k] through the C ABI."""
    import torch
    b, nq, hq, _ = q16.shape
    q_rot = torch.empty((b * nq, hq, 128), dtype=torch.float32, device="cuda")
    plan.rotate_queries(cache.consts, to_dev(q16.reshape(b * nq, hq, 128)), q_rot)
    out = torch.full((b, hq, nq, n_k), float("nan"), dtype=torch.float32, device="cuda")
    plan.key_logits(cache.consts, q_rot.view(b, nq, hq, 128), cache.k_codes, cache.k_norms, cache.capacity,
                    t0, n_k, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _case(bg, cid, seq_len, batch, n_q, t0, n_k, bits=None, avg=None, q_start=0):
    import torch
    cfg = synth.small(cid, seq_len=seq_len, batch=batch)
    avg = cfg.k_bits if avg is None else avg
    if bits is None:
        q_cal, k_cal = synth.calibration(cfg)
        _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, avg, cfg.pairing)
    plan = bg.Plan(bits, avg, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed, pairing=cfg.pairing)
    cache = bg.Cache(plan, batch, seq_len, device="cuda")
    ks = np.stack([synth.keys(cfg, seq=s, count=seq_len) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=seq_len) for s in range(batch)])
    cache.encode(to_dev(ks), to_dev(vs), 0)
    torch.cuda.synchronize()
    qs = np.stack([synth.queries(cfg, seq=s, start=q_start, count=n_q) for s in range(batch)])  # [b, n_q, Hq, 128]
    got = _library_logits(bg, plan, cache, qs, t0, n_k)
    return cfg, bits, ks, vs, qs, got


def _oracle_logits(cfg, bits, ks, qs, t0, n_k):
    b, nq, hq, _ = qs.shape
    ref = np.zeros((b, hq, nq, n_k))
    bound = np.zeros_like(ref)
    for s in range(b):
        for kvh in range(cfg.n_kv_heads):
            head = OracleHead(ks[s, :, kvh], np.zeros_like(ks[s, :, kvh]), bits[kvh], 1, cfg.seed, 0, kvh,
                              cfg.pairing)
            kh = head.k_hat()[t0:t0 + n_k]                                   # [n_k, 128] float64
            for h in range(kvh * cfg.group, (kvh + 1) * cfg.group):
                q = qs[s, :, h].astype(np.float64)                          # [n_q, 128]
                ref[s, h] = q @ kh.T
                bound[s, h] = np.outer(np.linalg.norm(q, axis=1), np.linalg.norm(kh, axis=1))
    return ref, bound


@pytest.mark.parametrize("cid,seq_len,batch,n_q,t0,n_k", [
    (1, 300, 1, 3, 0, 300),        # several tiles and a ragged tail
    (2, 257, 2, 2, 37, 200),       # offset range that starts and ends inside tiles
    (3, 130, 1, 5, 64, 66),        # G = 4, range starting on a tile boundary
    (5, 200, 1, 1, 199, 1),        # one token
])
def test_key_logits_match_oracle(bg, cid, seq_len, batch, n_q, t0, n_k):
    log("key logits config %d T=%d batch %d n_q %d range [%d, %d)" % (cid, seq_len, batch, n_q, t0, t0 + n_k))
    cfg, bits, ks, _, qs, got = _case(bg, cid, seq_len, batch, n_q, t0, n_k)
    ref, bound = _oracle_logits(cfg, bits, ks, qs, t0, n_k)
    assert np.all(np.isfinite(got))
    # fp32 products and sums of 128 terms, fp32 rotated queries: within 1e-5 of the Cauchy-Schwarz bound
    err = np.abs(got - ref)
    assert np.all(err <= 1e-5 * bound + 1e-30), float((err / np.maximum(bound, 1e-30)).max())


def test_key_logits_uniform_and_zero_bits(bg):
    """Uniform TQ-MSE (every block at the same width) and a plan without key bits (logits 0)."""
    cfg = synth.small(2, seq_len=100)
    for w in (2, 0):
        bits = np.full((cfg.n_kv_heads, 64), w, np.int8)
        log("key logits uniform width %d" % w)
        cfg_, bits_, ks, _, qs, got = _case(bg, 2, 100, 1, 2, 0, 100, bits=bits, avg=w)
        ref, bound = _oracle_logits(cfg_, bits_, ks, qs, 0, 100)
        if w == 0:
            assert np.all(got == 0)
        else:
            assert np.all(np.abs(got - ref) <= 1e-5 * bound + 1e-30)


def test_key_logits_rejects_bad_ranges(bg):
    import torch
    cfg = synth.small(1, seq_len=64)
    bits = np.full((cfg.n_kv_heads, 64), 2, np.int8)
    plan = bg.Plan(bits, 2, 2, cfg.n_q_heads)
    cache = bg.Cache(plan, 1, 64, device="cuda")
    q_rot = torch.zeros((1, 1, cfg.n_q_heads, 128), dtype=torch.float32, device="cuda")
    for t0, n_k in ((-1, 4), (10, 60), (0, 65)):
        out = torch.zeros((1, cfg.n_q_heads, 1, max(n_k, 0)), dtype=torch.float32, device="cuda")
        with pytest.raises(bg.BgtqError):
            plan.key_logits(cache.consts, q_rot, cache.k_codes, cache.k_norms, 64, t0, n_k, out)


def test_layer_mae_from_library_matches_oracle(bg):
    """The per-layer RoPE-logit MAE (causal pairs of the last M positions, unscaled logits) taken from
    the library's logits equals the oracle's MAE for Block-GTQ and uniform TQ-MSE at 2 and 3 bits."""
    cid, seq_len, m = 2, 512, 256
    cfg = synth.small(cid, seq_len=seq_len)
    q_cal, k_cal = synth.calibration(cfg)
    ks = synth.keys(cfg, count=seq_len)
    causal = np.tril(np.ones((m, m), dtype=bool))
    for avg in (2, 3):
        _, gtq = ref_bits(q_cal, k_cal, cfg.n_kv_heads, avg, cfg.pairing)
        uni = np.full((cfg.n_kv_heads, 64), avg, np.int8)
        for name, bits in (("block-gtq", gtq), ("uniform", uni)):
            _, _, _, _, qb, got = _case(bg, cid, seq_len, 1, m, seq_len - m, m, bits=bits, avg=avg,
                                        q_start=seq_len - m)
            qs = qb[0]                                                       # [m, Hq, 128]
            exact = np.einsum("nhd,thd->hnt", qs.astype(np.float64),
                              np.repeat(ks[seq_len - m:], cfg.group, axis=1).astype(np.float64))
            lib_mae = np.abs(got[0] - exact)[:, causal].mean()
            k_hat = np.stack([OracleHead(ks[:, h], np.zeros_like(ks[:, h]), bits[h], 1, cfg.seed, 0, h,
                                         cfg.pairing).k_hat() for h in range(cfg.n_kv_heads)], axis=1)
            ref_mae = oracle.diagnostics.logit_mae(qs, ks[seq_len - m:], k_hat[seq_len - m:], cfg.group)
            log("%s %d bits: library MAE %.6f, oracle MAE %.6f" % (name, avg, lib_mae, ref_mae))
            assert abs(lib_mae - ref_mae) <= 1e-4 * ref_mae
