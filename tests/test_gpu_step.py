"""GPU parity of the fused decode step (bgtq_decode_step): appends one key and value per
sequence at pos[b] and attends over pos[b] + 1 tokens.  Checked against the float64 oracle
(bit-exact packed cache, attention within 2e-3 relative L2) and against the separate
encode + decode calls (identical bits)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import OracleHead, decode_gpu, gpu_arrays, log, ref_bits, rel_l2, to_dev

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


def _plan(bg, cfg):
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    return bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed, layer=0), bits


def _step(bg, plan, cache, q, k_new, v_new, pos, max_seq_len):
    import torch
    b = q.shape[0]
    out = torch.empty((b, plan.n_q_heads, 128), dtype=torch.int16, device="cuda")
    ws = torch.empty(plan.workspace_size(b, max_seq_len), dtype=torch.uint8, device="cuda")
    cache.step(to_dev(q), to_dev(k_new), to_dev(v_new), to_dev(np.asarray(pos, np.int32)), max_seq_len, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.float16).astype(np.float64)


@pytest.mark.parametrize("cid,hq", [(4, None), (2, None), (1, None), (4, 56)])  # 56 / 8: G = 7, padded
def test_decode_step_ragged_matches_oracle(bg, cid, hq):
    import torch
    prefix, capacity = 200, 320
    cfg = synth.small(cid, seq_len=prefix, batch=4, **({} if hq is None else {"n_q_heads": hq}))
    plan, bits = _plan(bg, cfg)
    cache = bg.Cache(plan, 4, capacity, device="cuda")
    ks = np.stack([synth.keys(cfg, seq=s, count=prefix) for s in range(4)])
    vs = np.stack([synth.values(cfg, seq=s, count=prefix) for s in range(4)])
    cache.encode(to_dev(ks), to_dev(vs), 0)
    pos = [prefix, 63, 0, -1]  # new token, overwrite at a tile end, overwrite token 0, no append
    k_new = np.stack([synth.keys(cfg, seq=s + 10, count=1)[0] for s in range(4)])
    v_new = np.stack([synth.values(cfg, seq=s + 10, count=1)[0] for s in range(4)])
    q = np.stack([synth.query(cfg, seq=s) for s in range(4)])
    max_seq_len = prefix + 1
    log("decode step config %d (G = %d) pos %s" % (cid, cfg.group, pos))
    got = _step(bg, plan, cache, q, k_new, v_new, pos, max_seq_len)
    for s in range(4):
        n_tok = max(prefix, pos[s] + 1)
        k_all, v_all = ks[s].copy(), vs[s].copy()
        if n_tok > prefix:
            k_all = np.concatenate([k_all, k_new[s][None]])
            v_all = np.concatenate([v_all, v_new[s][None]])
        elif pos[s] >= 0:
            k_all[pos[s]], v_all[pos[s]] = k_new[s], v_new[s]
        heads = [OracleHead(k_all[:, h], v_all[:, h], bits[h], cfg.v_bits, cfg.seed, 0, h)
                 for h in range(cfg.n_kv_heads)]
        for h in range(cfg.n_kv_heads):
            for name, g, e in zip(("k_codes", "k_norms", "v_codes", "v_norms"), gpu_arrays(cache, s, h),
                                  heads[h].packed(cache.tiles)):
                assert np.array_equal(g, e), (name, s, h)
        seq_len = min(pos[s] + 1, max_seq_len) if pos[s] >= 0 else 0
        if seq_len == 0:
            assert np.all(got[s] == 0.0)
            continue
        kh = np.stack([hd.k_hat() for hd in heads], axis=1)
        vh = np.stack([hd.v_hat() for hd in heads], axis=1)
        ref = oracle.decode_attention(q[s], kh, vh, seq_len)
        r = rel_l2(got[s], ref)
        assert r.max() <= TOL, (s, r.max())


def test_decode_step_equals_separate_calls(bg):
    import torch
    prefix, capacity = 700, 768
    cfg = synth.small(3, seq_len=prefix + 1)
    plan, _ = _plan(bg, cfg)
    caches = [bg.Cache(plan, 1, capacity, device="cuda") for _ in range(2)]
    k = synth.keys(cfg, count=prefix + 1)[None]
    v = synth.values(cfg, count=prefix + 1)[None]
    for c in caches:
        c.encode(to_dev(k[:, :prefix]), to_dev(v[:, :prefix]), 0)
    q = synth.query(cfg)[None]
    got = _step(bg, plan, caches[0], q, k[:, prefix], v[:, prefix], [prefix], prefix + 1)
    caches[1].encode(to_dev(k[:, prefix:]), to_dev(v[:, prefix:]), prefix)
    ref = decode_gpu(plan, caches[1], q, [prefix + 1], prefix + 1)
    torch.cuda.synchronize()
    for h in range(cfg.n_kv_heads):
        for g, e in zip(gpu_arrays(caches[0], 0, h), gpu_arrays(caches[1], 0, h)):
            assert np.array_equal(g, e)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("cid,n_sink,n_recent", [(4, 4, 128), (2, 64, 300), (1, 0, 64)])
def test_decode_step_buffered_equals_separate_calls(bg, cid, n_sink, n_recent):
    """bgtq_decode_step_buffered equals, bit for bit, the encode of the new token, its copy into
    the fp16 buffers (bgtq_buffer_append) and the buffered decode over T + 1 tokens; both
    buffers and both caches end up identical."""
    import torch
    prefix, capacity, batch = 500, 576, 2
    cfg = synth.small(cid, seq_len=prefix + 1, batch=batch)
    log("buffered decode step config %d sink %d recent %d" % (cid, n_sink, n_recent))
    plan, _ = _plan(bg, cfg)
    caches = [bg.Cache(plan, batch, capacity, device="cuda") for _ in range(2)]
    bufs = [bg.Buffer(batch, cfg.n_kv_heads, n_sink, n_recent, device="cuda") for _ in range(2)]
    ks = np.stack([synth.keys(cfg, seq=s, count=prefix + 1) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=prefix + 1) for s in range(batch)])
    for c, bf in zip(caches, bufs):
        c.encode(to_dev(ks[:, :prefix]), to_dev(vs[:, :prefix]), 0)
        bf.append(to_dev(ks[:, :prefix]), to_dev(vs[:, :prefix]), 0)
    q = to_dev(np.stack([synth.query(cfg, seq=s) for s in range(batch)]))
    k_new, v_new = to_dev(ks[:, prefix]), to_dev(vs[:, prefix])
    pos = to_dev(np.full(batch, prefix, np.int32))
    out_s = torch.empty((batch, cfg.n_q_heads, 128), dtype=torch.int16, device="cuda")
    out_r = torch.empty_like(out_s)
    ws = torch.empty(plan.workspace_size(batch, prefix + 1), dtype=torch.uint8, device="cuda")
    c0, c1 = caches
    plan.decode_step_buffered(c0.consts, q, k_new, v_new, pos, prefix + 1, c0.k_codes, c0.k_norms, c0.v_codes,
                              c0.v_norms, capacity, bufs[0], out_s, ws)
    c1.encode(to_dev(ks[:, prefix:]), to_dev(vs[:, prefix:]), prefix)
    bufs[1].append(to_dev(ks[:, prefix:]), to_dev(vs[:, prefix:]), prefix)
    plan.decode_attn_buffered(c1.consts, q, c1.k_codes, c1.k_norms, c1.v_codes, c1.v_norms, capacity,
                              to_dev(np.full(batch, prefix + 1, np.int32)), prefix + 1, bufs[1], out_r, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out_s.cpu().numpy(), out_r.cpu().numpy())
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        assert torch.equal(getattr(c0, name), getattr(c1, name)), name
    for name in ("k_sink", "v_sink", "k_recent", "v_recent"):
        a, b = getattr(bufs[0], name), getattr(bufs[1], name)
        assert (a is None and b is None) or torch.equal(a, b), name
