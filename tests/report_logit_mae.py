"""Per-layer RoPE-logit MAE of the quantised key cache on the five synthetic layers (a reported
diagnostic): Block-GTQ against uniform TQ-MSE at the same K budget, K-only at 2 and 3 bits per
coordinate, over the last M = 1024 positions of each layer's full context (queries drawn like the
keys, causal pairs, unscaled logits).

Without flags the MAE comes from the oracle's encode and dequantisation.  With --library (GPU) it
comes from the library's own output: the window's keys are encoded into a packed cache, the queries
rotated, and the logits read back from the cache by bgtq_key_logits; the oracle's MAE is printed
beside it.

Usage: python tests/report_logit_mae.py [--library]   (prints a markdown table)
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import oracle  # noqa: E402
import synth  # noqa: E402
from test_oracle_diagnostics import _layer_mae  # noqa: E402


def _library_layer_mae(bg, cfg, avg_bits, m):
    """MAE of Block-GTQ and uniform TQ-MSE from the library's logits over the last m positions."""
    import torch
    t = cfg.seq_len
    q_cal, k_cal = synth.calibration(cfg)
    e = oracle.energy(q_cal, k_cal, cfg.n_kv_heads)
    dist = oracle.distortion_table()
    keys = synth.keys(cfg, start=t - m, count=m)                     # [m, Hkv, 128] fp16
    qs = synth.queries(cfg, start=t - m, count=m)                    # [m, Hq, 128] fp16
    exact = np.einsum("nhd,thd->hnt", qs.astype(np.float64),
                      np.repeat(keys, cfg.group, axis=1).astype(np.float64))
    causal = np.tril(np.ones((m, m), dtype=bool))
    dev = torch.device("cuda:0")
    out = {}
    for name in ("block-gtq", "uniform"):
        bits = np.stack([oracle.greedy_allocate(e[h], avg_bits, dist) if name == "block-gtq"
                         else np.full(64, avg_bits, np.int8) for h in range(cfg.n_kv_heads)])
        plan = bg.Plan(bits, avg_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed, pairing=cfg.pairing)
        cache = bg.Cache(plan, 1, m, device=dev)
        k16 = torch.from_numpy(keys.view(np.int16)[None].copy()).to(dev)
        plan.encode_k(cache.consts, k16, m, 0, cache.k_codes, cache.k_norms)
        q_rot = torch.empty((m, cfg.n_q_heads, 128), dtype=torch.float32, device=dev)
        plan.rotate_queries(cache.consts, torch.from_numpy(qs.view(np.int16).copy()).to(dev), q_rot)
        logits = torch.empty((1, cfg.n_q_heads, m, m), dtype=torch.float32, device=dev)
        plan.key_logits(cache.consts, q_rot.view(1, m, cfg.n_q_heads, 128), cache.k_codes, cache.k_norms, m,
                        0, m, logits)
        torch.cuda.synchronize()
        got = logits[0].cpu().numpy().astype(np.float64)
        out[name] = float(np.abs(got - exact)[:, causal].mean())
        plan.close()
    return out


def main() -> int:
    m = 1024
    lib = "--library" in sys.argv[1:]
    bg = None
    if lib:
        import decode_attention_bgtq_amd as bg
        bg.load()
        print("| layer | context | K bits | Block-GTQ MAE (library) | uniform TQ-MSE MAE (library) | reduction "
              "| Block-GTQ MAE (oracle) | uniform MAE (oracle) |")
        print("|---|---|---|---|---|---|---|---|")
    else:
        print("| layer | context | K bits | Block-GTQ MAE | uniform TQ-MSE MAE | reduction |")
        print("|---|---|---|---|---|---|")
    for cid in (1, 2, 3, 4, 5):
        cfg = synth.CONFIGS[cid]
        for avg in (2, 3):
            r = _layer_mae(cfg, avg, m)
            bq, un = r["block-gtq"], r["uniform"]
            if lib:
                g = _library_layer_mae(bg, cfg, avg, m)
                print("| %s | %d | %d | %.4f | %.4f | %.1f%% | %.4f | %.4f |" % (
                    cfg.name, cfg.seq_len, avg, g["block-gtq"], g["uniform"],
                    100 * (g["uniform"] - g["block-gtq"]) / g["uniform"], bq, un), flush=True)
            else:
                print("| %s | %d | %d | %.4f | %.4f | %.1f%% |" % (cfg.name, cfg.seq_len, avg, bq, un,
                                                                    100 * (un - bq) / un), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
