"""Per-layer RoPE-logit MAE of the quantised key cache on the five synthetic layers (a reported
diagnostic; computed with the oracle only): Block-GTQ against uniform TQ-MSE at the same K budget,
K-only at 2 and 3 bits per coordinate, over the last M = 1024 positions of each layer's full context
(queries drawn like the keys, causal pairs, unscaled logits).  The library's packed codes are
bit-identical to the oracle's (GPU parity tests), so the numbers hold for the library's cache.

Usage: python tests/report_logit_mae.py   (prints a markdown table)
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import synth  # noqa: E402
from test_oracle_diagnostics import _layer_mae  # noqa: E402


def main() -> int:
    m = 1024
    print("| layer | context | K bits | Block-GTQ MAE | uniform TQ-MSE MAE | reduction |")
    print("|---|---|---|---|---|---|")
    for cid in (1, 2, 3, 4, 5):
        cfg = synth.CONFIGS[cid]
        for avg in (2, 3):
            r = _layer_mae(cfg, avg, m)
            bg, un = r["block-gtq"], r["uniform"]
            print("| %s | %d | %d | %.4f | %.4f | %.1f%% |" % (cfg.name, cfg.seq_len, avg, bg, un, 100 * (un - bg) / un),
                  flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
