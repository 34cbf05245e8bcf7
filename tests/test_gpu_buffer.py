"""GPU parity of the fp16 sink + recent-window variant (the Block-GTQ README's "withbuffer"
setting): the buffer copy is bit-exact, the buffered decode matches the oracle's
decode_attention_buffered within 2e-3 relative L2 per (sequence, query head)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import OracleHead, decode_gpu, log, ref_bits, rel_l2, to_dev

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


def _i16(t):
    return t.cpu().numpy().view(np.float16)


@pytest.mark.parametrize("n_sink,n_recent", [(4, 128), (0, 64), (64, 0), (3, 100)])
def test_buffer_append_bitexact(bg, n_sink, n_recent):
    import torch
    cfg = synth.small(4, seq_len=300, batch=2)
    k = np.stack([synth.keys(cfg, seq=s, count=300) for s in range(2)])
    v = np.stack([synth.values(cfg, seq=s, count=300) for s in range(2)])
    buf = bg.Buffer(2, cfg.n_kv_heads, n_sink, n_recent)
    for a, b in zip([0, 3, 100, 250, 299], [3, 100, 250, 299, 300]):
        buf.append(to_dev(k[:, a:b]), to_dev(v[:, a:b]), a)
    torch.cuda.synchronize()
    if n_sink:
        np.testing.assert_array_equal(_i16(buf.k_sink), k[:, :n_sink].transpose(0, 2, 1, 3))
        np.testing.assert_array_equal(_i16(buf.v_sink), v[:, :n_sink].transpose(0, 2, 1, 3))
    if n_recent:
        t = np.arange(300 - n_recent, 300)
        kr, vr = _i16(buf.k_recent), _i16(buf.v_recent)
        np.testing.assert_array_equal(kr[:, :, t % n_recent], k[:, t].transpose(0, 2, 1, 3))
        np.testing.assert_array_equal(vr[:, :, t % n_recent], v[:, t].transpose(0, 2, 1, 3))


def _buffered_case(bg, cfg, seq_lens, n_sink, n_recent, capacity=None):
    import torch
    batch = len(seq_lens)
    t_max = max(max(seq_lens), 1)
    capacity = capacity or t_max
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    cache = bg.Cache(plan, batch, capacity, device="cuda")
    ks = np.stack([synth.keys(cfg, seq=s, count=t_max) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=t_max) for s in range(batch)])
    cache.encode(to_dev(ks), to_dev(vs), 0)
    # each sequence's buffers hold its own last tokens: append sequence by sequence up to its length
    buf = bg.Buffer(batch, cfg.n_kv_heads, n_sink, n_recent)
    for s in range(batch):
        one = bg.Buffer(1, cfg.n_kv_heads, n_sink, n_recent)
        if seq_lens[s]:
            one.append(to_dev(ks[s:s + 1, :seq_lens[s]]), to_dev(vs[s:s + 1, :seq_lens[s]]), 0)
        for name in ("k_sink", "v_sink", "k_recent", "v_recent"):
            if getattr(buf, name) is not None:
                getattr(buf, name)[s].copy_(getattr(one, name)[0])
    torch.cuda.synchronize()
    q = np.stack([synth.query(cfg, seq=s) for s in range(batch)])
    got = decode_gpu(plan, cache, q, seq_lens, t_max, buf=buf)
    worst = 0.0
    for s in range(batch):
        if seq_lens[s] == 0:
            assert np.all(got[s] == 0.0)
            continue
        heads = [OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h)
                 for h in range(cfg.n_kv_heads)]
        kh = np.stack([x.k_hat() for x in heads], axis=1)
        vh = np.stack([x.v_hat() for x in heads], axis=1)
        ref = oracle.decode_attention_buffered(q[s], ks[s], vs[s], kh, vh, seq_lens[s], n_sink, n_recent)
        r = rel_l2(got[s], ref)
        worst = max(worst, float(r.max()))
        assert r.max() <= TOL, (s, r.max())
    log("buffered decode worst rel-L2 %.3e" % worst)
    return plan, cache, q, got


@pytest.mark.parametrize("cid,seq_len,n_sink,n_recent", [
    (1, 1000, 4, 128), (2, 2000, 4, 128), (3, 3000, 4, 128),
    (1, 100, 4, 128), (1, 132, 4, 128), (1, 133, 4, 128), (1, 1, 4, 128),
    (1, 700, 0, 128), (1, 700, 4, 0), (2, 900, 64, 300), (1, 64, 64, 0), (1, 65, 64, 0)])
def test_decode_buffered_matches_oracle(bg, cid, seq_len, n_sink, n_recent):
    log("buffered decode config %d T=%d sink %d recent %d" % (cid, seq_len, n_sink, n_recent))
    _buffered_case(bg, synth.small(cid, seq_len=seq_len), [seq_len], n_sink, n_recent)


def test_decode_buffered_ragged_batch(bg):
    cfg = synth.small(4, seq_len=1100, batch=5)
    log("buffered decode ragged batch")
    _buffered_case(bg, cfg, [0, 1, 130, 700, 1100], 4, 128, capacity=1152)


def test_decode_buffered_without_buffer_is_plain_decode(bg):
    """Zero counts: the buffered entry is the plain decode, to the bit."""
    cfg = synth.small(2, seq_len=500)
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads)
    cache = bg.Cache(plan, 1, 500, device="cuda")
    cache.encode(to_dev(synth.keys(cfg, count=500)[None]), to_dev(synth.values(cfg, count=500)[None]), 0)
    q = synth.query(cfg)[None]
    a = decode_gpu(plan, cache, q, [500], 500)
    b = decode_gpu(plan, cache, q, [500], 500, buf=bg.Buffer(1, cfg.n_kv_heads, 0, 0))
    assert np.array_equal(a, b)
