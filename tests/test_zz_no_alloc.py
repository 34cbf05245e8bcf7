"""bgtq_decode_attn_noalloc (split partials in the library's device scratch) against
bgtq_decode_attn (caller workspace): two calls in a row, the second on a smaller input,
each bit-identical to the workspace entry's output on the same inputs and within the decode
tolerance of the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import OracleHead, log, ref_bits, rel_l2, to_dev

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


def _case(bg, cid, batch, seq_len):
    import torch
    cfg = synth.small(cid, seq_len=seq_len, batch=batch)
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    cache = bg.Cache(plan, batch, seq_len, device="cuda")
    ks = np.stack([synth.keys(cfg, seq=s, count=seq_len) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=seq_len) for s in range(batch)])
    cache.encode(to_dev(ks), to_dev(vs), 0)
    q = np.stack([synth.query(cfg, seq=s) for s in range(batch)])
    lens = np.array([seq_len - 37 * s for s in range(batch)], np.int32)
    torch.cuda.synchronize()
    return cfg, bits, plan, cache, ks, vs, q, lens


def _run(bg, plan, cache, q, lens, noalloc):
    import torch
    out = torch.empty((q.shape[0], plan.n_q_heads, 128), dtype=torch.int16, device="cuda")
    args = (cache.consts, to_dev(q), cache.k_codes, cache.k_norms, cache.v_codes, cache.v_norms, cache.capacity,
            to_dev(lens), int(lens.max()))
    if noalloc:
        plan.decode_attn_noalloc(*args, out)
    else:
        ws = torch.empty(plan.workspace_size(q.shape[0], int(lens.max())), dtype=torch.uint8, device="cuda")
        plan.decode_attn(*args, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.float16).astype(np.float64)


def test_noalloc_matches_workspace_entry_two_calls(bg):
    """Call 1: 2 sequences x 5000 tokens (128K layer shape); call 2, right after on the same
    scratch: 1 sequence x 700 tokens (32K layer shape, G = 8).  Each equals the workspace
    entry bit for bit and the oracle within tolerance."""
    for cid, batch, t in ((3, 2, 5000), (2, 1, 700)):
        log("no-alloc decode: config %d, batch %d, T %d" % (cid, batch, t))
        cfg, bits, plan, cache, ks, vs, q, lens = _case(bg, cid, batch, t)
        got = _run(bg, plan, cache, q, lens, noalloc=True)
        ref_ws = _run(bg, plan, cache, q, lens, noalloc=False)
        assert np.array_equal(got, ref_ws)
        for s in range(batch):
            kh = np.stack([OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h).k_hat()
                           for h in range(cfg.n_kv_heads)], axis=1)
            vh = np.stack([OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h).v_hat()
                           for h in range(cfg.n_kv_heads)], axis=1)
            ref = oracle.decode_attention(q[s], kh, vh, int(lens[s]))
            r = rel_l2(got[s], ref)
            log("no-alloc decode: sequence %d worst rel-L2 %.3e" % (s, r.max()))
            assert r.max() <= TOL


def test_noalloc_rejects_partials_beyond_the_scratch(bg):
    """255 sequences x 32 query heads of partials (4.3 MB) exceed the 4 MiB scratch: EWORKSPACE,
    nothing launched."""
    cfg = synth.small(3, seq_len=64)
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads)
    assert plan.workspace_size(255, 64) > bg.load().bgtq_noalloc_scratch_bytes()
    lib = bg.load()
    st = lib.bgtq_decode_attn_noalloc(plan.handle, 256, 256, 256, 256, 256, 256, 64, 256, 255, 64, 0.1, 256, None)
    assert st == bg.EWORKSPACE
