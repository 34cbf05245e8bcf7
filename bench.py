"""Benchmark of the Block-GTQ packed-KV decode path on one MI355X.

One step = one decode-attention call (bgtq_decode_attn: the query preparation
kernel, the decode kernel that streams the packed cache, then the split merge)
of the 128K Llama-3.1-8B-shaped layer (batch 1, 8 KV / 32 query heads, K2V2)
over the T+1 cached tokens.  The serving step (bgtq_decode_step: the new
token's key and value appended at position T, then the decode) is timed as
well and reported under "serving_step".
Calibration energy, allocation, plan creation and the full 128K prefill
encode run once before the timed region and are reported as separate fields,
and so does the fp16 baseline: the same keys and values uncompressed, decoded
by bgtq_fp16_decode_attn (same split-sequence structure) over the same tokens.
The other four synthetic layers (tiny 4K head, 32K Qwen-shaped, 16 x 32K
batched, 512K with a 4096-token append) are measured the same way and reported
under "configs".

value = algorithmic packed bytes read per step (codes + present fp16 norms)
/ step time.  The packed cache is replicated (>= 1 GiB in total), and so is
the plan's constant image (one copy per replica, as the layers of a model
would each have their own); steps rotate over the replicas so that reads come
from HBM, not the 256 MB Infinity Cache.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-KV decode attn GB/s (% HBM peak), ms/step @128K; encode keys/s"
HBM_PEAK_GBPS = 8000.0
FP64_PEAK_TFLOPS = 78.6
STREAM_KERNEL = "decode_kernel"
DTYPE = "fp16 and fp32 operands, fp32 accumulate"


def log(msg: str) -> None:
    print("[bench %s] %s" % (time.strftime("%H:%M:%S"), msg), file=sys.stderr, flush=True)


KERNEL_SOURCES = ("decode.hip", "prep.h", "merge.h", "device.h", "internal.h")


def kernel_source_hash() -> str:
    """SHA-256 prefix of the sources the decode kernel is compiled from."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "decode_attention_bgtq_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(cid: int):
    """Per-launch HBM bytes of the decode kernel from committed counter runs, if still valid."""
    p = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    rec = d.get("configs", {}).get(str(cid))
    if not rec or d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(cfg, bits, n_heads: int):
    """The oracle's decode (explicit dequantisation + float64 softmax attention) on a sample."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    import synth
    t = cfg.seq_len
    q = synth.query(cfg)
    n_heads = min(n_heads, cfg.n_kv_heads)
    k_all = synth.keys(cfg, count=t)
    v_all = synth.values(cfg, count=t)
    heads, step_bytes = [], 0
    for h in range(n_heads):  # the oracle's packed codes of the sample (setup, not timed)
        kc, kn = oracle.encode_k(k_all[:, h], bits[h], cfg.seed, 0, h)
        vc, vn = oracle.encode_v(v_all[:, h], cfg.v_bits, cfg.seed, 0, h)
        heads.append((h, kc, kn, vc, vn))
        n_groups = len([w for w in (1, 2, 3, 4) if np.any(bits[h] == w)])
        step_bytes += t * (16 * cfg.k_bits + 2 * n_groups + 16 * cfg.v_bits + 2)
    del k_all, v_all

    def one_pass():
        t0 = time.perf_counter()
        for h, kc, kn, vc, vn in heads:
            kh = oracle.dequant_k(kc, kn, bits[h], cfg.seed, 0, h)
            vh = oracle.dequant_v(vc, vn, cfg.v_bits, cfg.seed, 0, h)
            for hh in range(h * cfg.group, (h + 1) * cfg.group):
                oracle.softmax_attention(q[hh].astype(np.float64), kh, vh, 1 / math.sqrt(128))
        return time.perf_counter() - t0

    # repeated passes over the sample until about 10 s of CPU work (at most 30 passes)
    times = [one_pass()]
    while sum(times) < 10.0 and len(times) < 30:
        times.append(one_pass())
    med = float(np.median(times))
    log("cpu baseline: %d passes, median %.3f s per pass" % (len(times), med))
    return {"value": step_bytes / med / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": "float64 oracle decode (dequantise + softmax attention) of %d of %d KV heads x %d tokens "
                      "(all %d query heads of those KV heads); packed bytes of the sample / median wall time "
                      "of %d passes (%.1f s of CPU work)" %
                      (n_heads, cfg.n_kv_heads, t, n_heads * cfg.group, len(times), sum(times))}


def traffic_from(fetch_dir: str, write_dir: str, cid: int, packed: int | None, out_path: str) -> int:
    """Turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE) into
    profiles/decode_kernel_traffic.json.  Both counters are scaled by what they read for the
    1 GiB device copy of the copy probe (1 GiB read, 1 GiB written)."""
    import csv
    import glob

    def rows(d):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit("no counter_collection.csv under %s" % d)
        return list(csv.DictReader(open(f[0])))

    def per_kernel(rs, counter):
        copy, stream = [], []
        for r in rs:
            if r["Counter_Name"] != counter:
                continue
            dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            if "copyBuffer" in r["Kernel_Name"]:
                copy.append((dur, float(r["Counter_Value"])))
            elif ("bgtq::%s<" % STREAM_KERNEL) in r["Kernel_Name"]:  # not the fp16 baseline's kernel
                stream.append(float(r["Counter_Value"]))
        top = max(d for d, _ in copy)
        big = [v for d, v in copy if d >= top / 2]  # the 1 GiB copies
        return sum(big) / len(big), sum(stream) / len(stream), len(big), len(stream)

    fc, fs, nfc, nfs = per_kernel(rows(fetch_dir), "FETCH_SIZE")
    wc, ws, nwc, nws = per_kernel(rows(write_dir), "WRITE_SIZE")
    gib = float(1 << 30)
    rscale, wscale = gib / (fc * 1024), gib / (wc * 1024)
    rec = {"fetch_bytes": round(fs * 1024 * rscale), "write_bytes": round(ws * 1024 * wscale),
           "fetch_kib_raw": fs, "write_kib_raw": ws, "launches": [nfs, nws]}
    rec["hbm_bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    if packed:
        rec["algorithmic_bytes_per_launch"] = packed
    out = {"kernel": STREAM_KERNEL, "kernel_source_sha256_16": kernel_source_hash(),
           "copy_scale": {"fetch": rscale, "write": wscale, "copy_fetch_kib_raw": fc, "copy_write_kib_raw": wc,
                          "copies": [nfc, nwc]},
           "configs": {str(cid): rec}}
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


class Timer:
    """Event timing of enqueued calls on torch's current stream (the library's calls go to it)."""

    def __init__(self, torch):
        self.torch = torch
        self.spin = getattr(torch.cuda, "_sleep", None)

    def ev(self):
        return self.torch.cuda.Event(enable_timing=True)

    def _hold(self):
        # a short GPU spin, so that the host has queued every call before the GPU reaches them
        self.torch.cuda.synchronize()
        if self.spin is not None:
            self.spin(int(30e6))

    def rounds(self, fn, steps, i0=0):
        """Mean ms per call over `steps` calls in rounds of at most 100, no events between calls;
        also the host enqueue time per call."""
        per_round = min(steps, 100)
        n_rounds = max(1, steps // per_round)
        tot_ms, host_s, n = 0.0, 0.0, 0
        for _ in range(n_rounds):
            self._hold()
            s0, s1 = self.ev(), self.ev()
            s0.record()
            th = time.perf_counter()
            for i in range(per_round):
                fn(i0 + n + i)
            host_s += time.perf_counter() - th
            s1.record()
            self.torch.cuda.synchronize()
            tot_ms += s0.elapsed_time(s1)
            n += per_round
        return tot_ms / n, host_s * 1e3 / n, n

    def per_call(self, fn, steps, i0=0):
        """Duration of each of `steps` back-to-back calls (an event between consecutive calls)."""
        out = []
        per_round = min(steps, 100)
        done = 0
        while done < steps:
            k = min(per_round, steps - done)
            self._hold()
            evs = [self.ev() for _ in range(k + 1)]
            evs[0].record()
            for i in range(k):
                fn(i0 + done + i)
                evs[i + 1].record()
            self.torch.cuda.synchronize()
            out += [evs[i].elapsed_time(evs[i + 1]) for i in range(k)]
            done += k
        return out


def kernel_ms(bg, timer, fn, steps):
    """Mean duration of the decode kernel: the library's HIP events bound to every decode-kernel
    launch (hipExtLaunchKernel on the launch stream, so the elapsed time is the kernel's own
    start-to-end time), in a pass of its own because event timing can slow the dispatch of the
    launches around it."""
    bg.profile_enable(True)
    bg.profile_read()
    timer.rounds(fn, steps)
    bg.profile_enable(False)
    total, launches = bg.profile_read()
    return total / max(launches, 1), launches


def encode_flops(bits) -> tuple[float, float]:
    """fp64 flops per token-head of the encode's rotations (2 d_g^2 per key group, 2 x 128^2 for the
    value), averaged over the KV heads; the norms and threshold counts are not counted."""
    fk = [sum(2.0 * (2 * int((row == w).sum())) ** 2 for w in (1, 2, 3, 4)) for row in bits]
    return float(np.mean(fk)), 2.0 * 128 * 128


class Layer:
    """One synthetic layer resident in HBM: plan, prefill-encoded packed cache (capacity T plus the
    workload's append), replicas of the cache and of the constant image, the query and new token."""

    def __init__(self, bg, torch, cfg, dev, replica_bytes, keep_fp16=False):
        import synth
        self.cfg = cfg
        b, t, hkv, hq = cfg.batch, cfg.seq_len, cfg.n_kv_heads, cfg.n_q_heads
        timer = Timer(torch)

        def to_dev(a):
            a = np.ascontiguousarray(a)
            return torch.from_numpy(a.view(np.int16) if a.dtype == np.float16 else a).to(dev)

        self.to_dev = to_dev
        # ---- one-time rows: energy, allocation, plan
        q_cal, k_cal = synth.calibration(cfg)
        qc, kc = to_dev(q_cal), to_dev(k_cal)
        e_dev = torch.empty((hkv, 64), dtype=torch.float64, device=dev)
        bits_dev = torch.empty((hkv, 64), dtype=torch.int8, device=dev)
        bg.energy(qc, kc, hkv, e_dev)
        bg.allocate_device(e_dev, cfg.k_bits, bits_dev)
        torch.cuda.synchronize()
        e0, e1, e2 = timer.ev(), timer.ev(), timer.ev()
        e0.record()
        for _ in range(10):
            bg.energy(qc, kc, hkv, e_dev)
        e1.record()
        for _ in range(10):
            bg.allocate_device(e_dev, cfg.k_bits, bits_dev)
        e2.record()
        torch.cuda.synchronize()
        self.energy_us = e0.elapsed_time(e1) * 100.0
        self.energy_bytes = q_cal.size * 2 + k_cal.size * 2
        self.alloc_us = e1.elapsed_time(e2) * 100.0
        self.bits = bits_dev.cpu().numpy()
        th = time.perf_counter()
        bits_host = bg.allocate(e_dev.cpu().numpy(), cfg.k_bits)
        self.alloc_host_us = (time.perf_counter() - th) * 1e6
        assert np.array_equal(bits_host, self.bits), "host and device allocations differ"
        tp = time.perf_counter()
        self.plan = plan = bg.Plan(self.bits, cfg.k_bits, cfg.v_bits, hq, seed=cfg.seed, layer=0)
        self.plan_ms = (time.perf_counter() - tp) * 1e3
        del qc, kc

        # ---- prefill encode of the whole context (timed once more after a first pass)
        self.cap = cap = t + max(64, cfg.append)
        self.cache = cache = bg.Cache(plan, b, cap, device=dev)
        log("%s: generating %d x %d tokens" % (cfg.name, b, t))
        kd = to_dev(np.stack([synth.keys(cfg, seq=s, count=t) for s in range(b)]))
        vd = to_dev(np.stack([synth.values(cfg, seq=s, count=t) for s in range(b)]))
        cache.encode(kd, vd, 0)
        torch.cuda.synchronize()
        e0, e1, e2, e3 = timer.ev(), timer.ev(), timer.ev(), timer.ev()
        e0.record()
        plan.encode_k(cache.consts, kd, cap, 0, cache.k_codes, cache.k_norms)
        e1.record()
        plan.encode_v(cache.consts, vd, cap, 0, cache.v_codes, cache.v_norms)
        e2.record()
        cache.encode_kv(kd, vd, 0)  # keys and values in one call (the same codes)
        e3.record()
        torch.cuda.synchronize()
        self.enc_k_s, self.enc_v_s = e0.elapsed_time(e1) / 1e3, e1.elapsed_time(e2) / 1e3
        self.enc_kv_s = e2.elapsed_time(e3) / 1e3
        self.token_heads = b * t * hkv
        self.kd, self.vd = (kd, vd) if keep_fp16 else (None, None)
        del kd, vd
        # ---- the workload's append (new tokens at positions T ..), encoded into the same cache
        self.append = None
        if cfg.append > 0:
            ka = to_dev(np.stack([synth.keys(cfg, seq=s, start=t, count=cfg.append) for s in range(b)]))
            va = to_dev(np.stack([synth.values(cfg, seq=s, start=t, count=cfg.append) for s in range(b)]))
            plan.encode_k(cache.consts, ka, cap, t, cache.k_codes, cache.k_norms)
            plan.encode_v(cache.consts, va, cap, t, cache.v_codes, cache.v_norms)
            plan.encode_kv(cache.consts, ka, va, cap, t, cache.k_codes, cache.k_norms, cache.v_codes,
                           cache.v_norms)
            torch.cuda.synchronize()
            # (re-encoding the same tokens writes the same codes: the cache stays as it was)
            n_kv = 10
            a0, a1, a2, a3 = timer.ev(), timer.ev(), timer.ev(), timer.ev()
            a0.record()
            plan.encode_k(cache.consts, ka, cap, t, cache.k_codes, cache.k_norms)
            a1.record()
            plan.encode_v(cache.consts, va, cap, t, cache.v_codes, cache.v_norms)
            a2.record()
            for _ in range(n_kv):
                plan.encode_kv(cache.consts, ka, va, cap, t, cache.k_codes, cache.k_norms, cache.v_codes,
                               cache.v_norms)
            a3.record()
            torch.cuda.synchronize()
            ak, av = a0.elapsed_time(a1) / 1e3, a1.elapsed_time(a2) / 1e3
            akv = a2.elapsed_time(a3) / 1e3 / n_kv
            ath = b * cfg.append * hkv
            fk, fv = encode_flops(self.bits)
            self.append = {"what": "bgtq_encode_kv: the new keys and values in one call (mean of %d)" % n_kv,
                           "tokens": cfg.append, "at": t, "k_and_v": round(ath / akv), "us": round(akv * 1e6, 2),
                           "fp64_frac": round(ath * (fk + fv) / akv / 1e12 / FP64_PEAK_TFLOPS, 4),
                           "two_calls_us": round((ak + av) * 1e6, 2), "k": round(ath / ak), "v": round(ath / av)}
            log("%s: append of %d tokens at %d: %.1f us in one call (%.0f M token-heads/s); "
                "encode_k + encode_v %.1f us" % (cfg.name, cfg.append, t, akv * 1e6, ath / akv / 1e6,
                                                 (ak + av) * 1e6))
            del ka, va

        # ---- the appended token and the query (position T), written into every replica
        cfg1 = dataclasses.replace(cfg, append=1)
        self.k_new = to_dev(np.stack([synth.keys(cfg1, seq=s, start=t, count=1) for s in range(b)]))
        self.v_new = to_dev(np.stack([synth.values(cfg1, seq=s, start=t, count=1) for s in range(b)]))
        self.q = to_dev(np.stack([synth.query(cfg, seq=s, pos=t) for s in range(b)]))
        self.packed = cache.packed_bytes(t + 1)
        self.n_rep = n_rep = max(1, math.ceil(replica_bytes / self.packed))
        log("%s: packed bytes/step %.1f MB; %d replicas" % (cfg.name, self.packed / 1e6, n_rep))
        self.reps = [(cache.consts, cache.k_codes, cache.k_norms, cache.v_codes, cache.v_norms)]
        for _ in range(n_rep - 1):
            self.reps.append(tuple(x.clone() for x in self.reps[0]))
        self.out = torch.empty((b, hq, 128), dtype=torch.int16, device=dev)
        self.ws = torch.empty(plan.workspace_size(b, t + 1), dtype=torch.uint8, device=dev)
        self.pos = torch.full((b,), t, dtype=torch.int32, device=dev)
        self.seq_lens = torch.full((b,), t + 1, dtype=torch.int32, device=dev)
        for i in range(n_rep):  # every replica holds token t before the timed decode calls
            self.serve(i)
        torch.cuda.synchronize()

    def attn(self, i):  # one decode-attention call over T + 1 tokens
        c_, kc_, kn_, vc_, vn_ = self.reps[i % self.n_rep]
        t = self.cfg.seq_len
        self.plan.decode_attn(c_, self.q, kc_, kn_, vc_, vn_, self.cap, self.seq_lens, t + 1, self.out, self.ws)

    def serve(self, i):  # one serving step: append the new key / value at T, then attend
        c_, kc_, kn_, vc_, vn_ = self.reps[i % self.n_rep]
        t = self.cfg.seq_len
        self.plan.decode_step(c_, self.q, self.k_new, self.v_new, self.pos, t + 1, kc_, kn_, vc_, vn_, self.cap,
                              self.out, self.ws)

    def record(self, bg, timer, steps, warmup):
        """Decode timing, kernel roofline, percentiles, serving step, encode and append rates."""
        for i in range(warmup):
            self.attn(i)
            self.serve(i)
        step_ms, host_ms, n = timer.rounds(self.attn, steps)
        calls = timer.per_call(self.attn, steps)
        serve_ms = timer.rounds(self.serve, steps)[0]
        k_ms, launches = kernel_ms(bg, timer, self.attn, steps)
        fk, fv = encode_flops(self.bits)
        th = self.token_heads
        enc_s = self.enc_kv_s
        cfg = self.cfg
        rec = {
            "workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seq_len, "n_kv_heads": cfg.n_kv_heads,
            "n_q_heads": cfg.n_q_heads, "k_bits": cfg.k_bits, "v_bits": cfg.v_bits,
            "packed_bytes_per_step": self.packed, "decode_ms": round(step_ms, 5),
            "decode_GBps": round(self.packed / (step_ms / 1e3) / 1e9, 2),
            "decode_hbm_peak_frac": round(self.packed / (step_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "decode_ms_p10_p50_p90": [round(float(x), 5) for x in np.percentile(calls, [10, 50, 90])],
            "kernel_ms": round(k_ms, 5),
            "kernel_frac": round(self.packed / (k_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
            "serving_step_ms": round(serve_ms, 5),
            "encode": {"what": "bgtq_encode_kv of the whole context (keys and values in one call); k and v: "
                               "bgtq_encode_k and bgtq_encode_v alone",
                       "token_heads_per_s": round(th / enc_s),
                       "two_calls": round(th / (self.enc_k_s + self.enc_v_s)), "k": round(th / self.enc_k_s),
                       "v": round(th / self.enc_v_s), "tokens": cfg.batch * cfg.seq_len,
                       "fp64_flops_per_token_head": {"k": round(fk), "v": round(fv)},
                       "fp64_frac": round(th * (fk + fv) / enc_s / 1e12 / FP64_PEAK_TFLOPS, 4)},
            "energy": {"us": round(self.energy_us, 2), "bytes": self.energy_bytes,
                       "hbm_peak_frac": round(self.energy_bytes / (self.energy_us / 1e6) / 1e9 / HBM_PEAK_GBPS, 5)},
            "append": self.append,
        }
        log("%s: decode %.4f ms (%.0f GB/s), kernel %.4f ms (frac %.3f, %d launches), p10/50/90 %s, "
            "serving step %.4f ms, host enqueue %.4f ms/call" % (
                cfg.name, step_ms, self.packed / (step_ms / 1e3) / 1e9, k_ms, rec["kernel_frac"], launches,
                rec["decode_ms_p10_p50_p90"], serve_ms, host_ms))
        return rec, step_ms, serve_ms, k_ms, calls, n

    def free(self):
        self.reps = self.kd = self.vd = None
        self.plan.close()


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--replica-bytes", type=float, default=1.1e9)
    ap.add_argument("--cpu-heads", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="measure only the main workload (for profiler runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/decode_kernel_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--packed-bytes", type=int, default=None)
    ap.add_argument("--traffic-out", default=os.path.join(ROOT, "profiles", "decode_kernel_traffic.json"))
    args = ap.parse_args()
    if args.traffic_from:
        return traffic_from(args.traffic_from[0], args.traffic_from[1], args.config, args.packed_bytes,
                            args.traffic_out)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: the decode path has no multi-GPU mode here (KV heads, "
              "sequences and token ranges would shard with one partial merge); run with --gpus 1",
              file=sys.stderr)
        return 2

    import torch
    import decode_attention_bgtq_amd as bg
    import synth

    if not os.path.exists(bg.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    cfg = synth.CONFIGS[args.config]
    b, t, hkv, hq = cfg.batch, cfg.seq_len, cfg.n_kv_heads, cfg.n_q_heads
    log("config %d %s: batch %d, T %d, %d/%d heads, K%dV%d" % (cfg.cid, cfg.name, b, t, hkv, hq, cfg.k_bits,
                                                              cfg.v_bits))
    timer = Timer(torch)
    lay = Layer(bg, torch, cfg, dev, args.replica_bytes, keep_fp16=True)
    main_rec, step_ms, serve_ms, kern_ms, calls, n_steps = lay.record(bg, timer, args.steps, args.warmup)
    packed = lay.packed
    value = packed / (step_ms / 1e3) / 1e9
    achieved = packed / (kern_ms / 1e3) / 1e9

    # ---- the fp16 sink + recent-window variant (4 + 128 tokens in fp16, the rest packed)
    buf = bg.Buffer(b, hkv, 4, 128, device=dev)
    buf.append(lay.kd, lay.vd, 0)
    buf.append(lay.k_new, lay.v_new, t)

    def attn_buf(i):
        c_, kc_, kn_, vc_, vn_ = lay.reps[i % lay.n_rep]
        lay.plan.decode_attn_buffered(c_, lay.q, kc_, kn_, vc_, vn_, lay.cap, lay.seq_lens, t + 1, buf, lay.out,
                                      lay.ws)

    for i in range(max(5, args.warmup // 5)):
        attn_buf(i)
    buf_ms = timer.rounds(attn_buf, args.steps)[0]
    log("buffered decode (4 sink + 128 recent fp16 tokens) %.4f ms" % buf_ms)

    def serve_buf(i):  # the serving step with the buffers: the new token at T into the cache and the buffers
        c_, kc_, kn_, vc_, vn_ = lay.reps[i % lay.n_rep]
        lay.plan.decode_step_buffered(c_, lay.q, lay.k_new, lay.v_new, lay.pos, t + 1, kc_, kn_, vc_, vn_, lay.cap,
                                      buf, lay.out, lay.ws)

    for i in range(max(5, args.warmup // 5)):
        serve_buf(i)
    serve_buf_ms = timer.rounds(serve_buf, args.steps)[0]
    log("buffered serving step %.4f ms" % serve_buf_ms)
    del buf

    # ---- the paged layout: each replica read as a pool of pages [Hkv][tiles] through a shuffled
    # block table (one sequence), the same bytes per call
    paged_ms = None
    if b == 1:
        table = torch.from_numpy(np.random.default_rng(0).permutation(lay.cache.tiles).astype(np.int32)[None]).to(dev)

        class _Pool:
            def __init__(self, arrs):
                self.consts, self.k_codes, self.k_norms, self.v_codes, self.v_norms = arrs

            def desc(self):
                return bg._Pages(table.data_ptr(), lay.cache.tiles, lay.cache.tiles)

        pools = [_Pool(r) for r in lay.reps]

        def attn_paged(i):
            pl = pools[i % lay.n_rep]
            lay.plan.decode_attn_paged(pl.consts, lay.q, pl, lay.seq_lens, t + 1, lay.out, lay.ws)

        for i in range(max(5, args.warmup // 5)):
            attn_paged(i)
        paged_ms = timer.rounds(attn_paged, args.steps)[0]
        log("paged decode (shuffled block table) %.4f ms" % paged_ms)

    # ---- fp16 baseline: the same keys and values uncompressed, the same split-sequence decode
    # (bgtq_fp16_decode_attn) over the same t + 1 tokens, replicated against the Infinity Cache
    reps_main = lay.reps
    lay.reps = None
    del reps_main
    kf = torch.zeros((b, lay.cap, hkv, 128), dtype=torch.int16, device=dev)
    vf = torch.zeros_like(kf)
    kf[:, :t] = lay.kd
    vf[:, :t] = lay.vd
    kf[:, t] = lay.k_new[:, 0]
    vf[:, t] = lay.v_new[:, 0]
    lay.kd = lay.vd = None
    fp16_bytes = b * (t + 1) * hkv * 128 * 2 * 2
    n_rep16 = max(1, math.ceil(args.replica_bytes / fp16_bytes))
    reps16 = [(kf, vf)] + [(kf.clone(), vf.clone()) for _ in range(n_rep16 - 1)]
    ws16 = torch.empty(bg.fp16_workspace_size(b, hkv, hq, t + 1), dtype=torch.uint8, device=dev)

    def fp16_attn(i):
        kk, vv = reps16[i % n_rep16]
        bg.fp16_decode_attn(lay.q, kk, vv, lay.seq_lens, t + 1, lay.out, ws16)

    for i in range(max(5, args.warmup // 5)):
        fp16_attn(i)
    fp16_ms = timer.rounds(fp16_attn, max(100, args.steps // 5))[0]
    log("fp16 baseline %.4f ms (%.0f GB/s of fp16 K/V); packed decode %.2fx faster" %
        (fp16_ms, fp16_bytes / (fp16_ms / 1e3) / 1e9, fp16_ms / step_ms))
    del reps16, kf, vf

    # ---- copy probe: practical streaming ceiling (1 GiB read + 1 GiB write)
    src = torch.empty(1 << 28, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = timer.ev(), timer.ev()
    c0.record()
    for _ in range(10):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * src.numel() * 4 * 10 / (c0.elapsed_time(c1) / 1e3) / 1e9
    del src, dst

    # ---- the other synthetic layers, measured the same way (decode, kernel, encode, append)
    others = {}
    if not args.no_other_configs:
        for cid in sorted(synth.CONFIGS):
            if cid == cfg.cid:
                continue
            o = Layer(bg, torch, synth.CONFIGS[cid], dev, args.replica_bytes)
            others[str(cid)] = o.record(bg, timer, min(args.steps, 200), min(args.warmup, 20))[0]
            o.free()
            del o
            torch.cuda.empty_cache()

    traffic = load_traffic(cfg.cid)
    fk, fv = encode_flops(lay.bits)
    enc_s = lay.enc_kv_s
    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": n_steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
        "step_ms_p10_p50_p90": main_rec["decode_ms_p10_p50_p90"],
        "step_ms_percentiles_from": "per-call event times of %d back-to-back decode calls" % len(calls),
        "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": cfg.name, "batch": b, "seq_len": t, "n_kv_heads": hkv, "n_q_heads": hq,
                   "k_bits": cfg.k_bits, "v_bits": cfg.v_bits, "head_dim": 128, "cache_io": "packed codes + fp16 norms",
                   "query_io": "fp16", "accumulate": "fp32", "parallelism": "single GPU"},
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "serving_step": {"what": "bgtq_decode_step: the new token's key and value appended at position T, then "
                                 "decode attention over T + 1 tokens", "ms": round(serve_ms, 5),
                         "GBps": round(packed / (serve_ms / 1e3) / 1e9, 2)},
        "packed_bytes_per_step": packed,
        "paged_decode": {"what": "bgtq_decode_attn_paged: the same cache read as 64-token pages through a "
                                 "shuffled block table", "ms": None if paged_ms is None else round(paged_ms, 5)},
        "buffered_decode": {"what": "bgtq_decode_attn_buffered: 4 sink and 128 recent tokens from fp16 buffers, "
                                    "the rest from the packed cache, over the same t + 1 tokens; serving_step_ms: "
                                    "bgtq_decode_step_buffered (the new token into the cache and the buffers, "
                                    "then that decode)",
                            "ms": round(buf_ms, 5),
                            "serving_step_ms": round(serve_buf_ms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": STREAM_KERNEL, "kernel_ms": round(kern_ms, 5)},
        "append_token_heads_per_s": lay.append,
        "encode_token_heads_per_s": {"what": "prefill encode of the whole context: bgtq_encode_kv (keys and "
                                             "values in one call); k and v: bgtq_encode_k and bgtq_encode_v alone",
                                     "k_and_v": round(lay.token_heads / enc_s),
                                     "two_calls": round(lay.token_heads / (lay.enc_k_s + lay.enc_v_s)),
                                     "k": round(lay.token_heads / lay.enc_k_s),
                                     "v": round(lay.token_heads / lay.enc_v_s), "tokens": b * t,
                                     "roofline": {"bound": "fp64", "peak_TFLOPs": FP64_PEAK_TFLOPS,
                                                  "flops_per_token_head": round(fk + fv),
                                                  "frac": main_rec["encode"]["fp64_frac"]}},
        "fp16_baseline": {"what": "bgtq_fp16_decode_attn: the same keys and values uncompressed (fp16), the same "
                                  "split-sequence decode and merge, over the same t + 1 tokens",
                          "ms": round(fp16_ms, 5), "bytes_per_step": fp16_bytes,
                          "GBps": round(fp16_bytes / (fp16_ms / 1e3) / 1e9, 2),
                          "hbm_peak_frac": round(fp16_bytes / (fp16_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "packed_speedup": round(fp16_ms / step_ms, 3),
                          "packed_speedup_at_copy_ceiling": round(fp16_bytes / (copy_gbps * 1e9) * 1e3 / step_ms, 3),
                          "compression": round(fp16_bytes / packed, 3)},
        "copy_ceiling_GBps": round(copy_gbps, 1),
        "one_time": {"energy_us": round(lay.energy_us, 2), "energy_hbm_peak_frac": main_rec["energy"]["hbm_peak_frac"],
                     "allocate_device_us": round(lay.alloc_us, 2), "allocate_host_us": round(lay.alloc_host_us, 2),
                     "plan_host_ms": round(lay.plan_ms, 2)},
        "configs": others,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, lay.bits, args.cpu_heads)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
