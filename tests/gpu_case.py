"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI and the
oracle on the same seeded inputs.  Expected values come only from the oracle."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
import synth
from oracle import layout

TILE = 64


def log(msg: str) -> None:
    print("[%s] %s" % (time.strftime("%H:%M:%S"), msg), flush=True)


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def ref_bits(q_cal, k_cal, n_kv, avg, pairing="half"):
    e = oracle.energy(q_cal, k_cal, n_kv, pairing)
    dist = oracle.distortion_table()
    return e, np.stack([oracle.greedy_allocate(e[h], avg, dist) for h in range(n_kv)])


class OracleHead:
    """Oracle encode of one (sequence, KV head) over tokens [0, t)."""

    def __init__(self, k16, v16, bits_row, v_bits, seed, layer, kvh, pairing="half"):
        self.bits_row = bits_row
        self.v_bits = v_bits
        self.pairing = pairing
        self.kc, self.kn = oracle.encode_k(k16, bits_row, seed, layer, kvh, pairing=pairing)
        self.vc, self.vn = oracle.encode_v(v16, v_bits, seed, layer, kvh)
        self.seed, self.layer, self.kvh = seed, layer, kvh

    def packed(self, n_tiles):
        karr, knrm = layout.pack_k(self.kc, self.kn, self.bits_row, n_tiles)
        varr, vnrm = layout.pack_v(self.vc, self.vn, self.v_bits, n_tiles)
        return karr, knrm, varr, vnrm

    def k_hat(self):
        return oracle.dequant_k(self.kc, self.kn, self.bits_row, self.seed, self.layer, self.kvh,
                                pairing=self.pairing)

    def v_hat(self):
        return oracle.dequant_v(self.vc, self.vn, self.v_bits, self.seed, self.layer, self.kvh)


def gpu_arrays(cache, b, h):
    """(k_codes, k_norms, v_codes, v_norms) of one (sequence, KV head) as unsigned numpy arrays."""
    return (cache.k_codes[b, h].cpu().numpy().view(np.uint32),
            cache.k_norms[b, h].cpu().numpy().view(np.uint16),
            cache.v_codes[b, h].cpu().numpy().view(np.uint32),
            cache.v_norms[b, h].cpu().numpy().view(np.uint16))


def rel_l2(got, ref):
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return np.where(den > 0, num / np.maximum(den, 1e-300), num)


def decode_gpu(plan, cache, q16_batch, seq_lens, max_seq_len, scale=None, buf=None):
    """The packed decode through the C ABI (with ``buf``: the fp16 sink / recent-window variant)."""
    import torch
    b = q16_batch.shape[0]
    out = torch.empty((b, plan.n_q_heads, 128), dtype=torch.int16, device=dev())
    ws = torch.empty(plan.workspace_size(b, max_seq_len), dtype=torch.uint8, device=dev())
    args = (cache.consts, to_dev(q16_batch), cache.k_codes, cache.k_norms, cache.v_codes, cache.v_norms,
            cache.capacity, to_dev(np.asarray(seq_lens, np.int32)), max_seq_len)
    if buf is None:
        plan.decode_attn(*args, out, ws, softmax_scale=scale)
    else:
        plan.decode_attn_buffered(*args, buf, out, ws, softmax_scale=scale)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.float16).astype(np.float64)


__all__ = ["log", "dev", "to_dev", "ref_bits", "OracleHead", "gpu_arrays", "rel_l2", "decode_gpu",
           "synth", "sys"]
