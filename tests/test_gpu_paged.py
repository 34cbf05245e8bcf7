"""GPU parity of the paged packed cache: a pool of 64-token pages per KV head and a block
table.  Every page written by the paged encode equals the oracle's packed tile of the same
tokens, bit for bit; the paged decode equals the contiguous decode of the same tokens bit for
bit and the oracle within 2e-3 relative L2 per (sequence, query head)."""
import numpy as np
import pytest

import oracle
import synth
from gpu_case import OracleHead, dev, log, ref_bits, rel_l2, to_dev

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


def _pool_tile(arr, kvh, page):
    return arr[kvh, page].cpu().numpy()


@pytest.mark.parametrize("cid,seq_len,batch", [(4, 700, 3), (1, 1000, 1), (2, 300, 2)])
def test_paged_encode_and_decode(bg, cid, seq_len, batch):
    import torch
    cfg = synth.small(cid, seq_len=seq_len, batch=batch)
    log("paged config %d T=%d batch %d" % (cid, seq_len, batch))
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    n_tiles = (seq_len + 63) // 64
    max_pages = n_tiles + 1
    n_pages = batch * max_pages + 3
    rng = np.random.default_rng(cid)
    perm = rng.permutation(n_pages)
    table = perm[:batch * max_pages].reshape(batch, max_pages).astype(np.int32)
    pool = bg.PagedCache(plan, n_pages, table)
    cont = bg.Cache(plan, batch, seq_len)
    ks = np.stack([synth.keys(cfg, seq=s, count=seq_len) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=seq_len) for s in range(batch)])
    bounds = [0, 37, 42, 64, 101, seq_len] if seq_len > 101 else [0, seq_len]
    for a, b in zip(bounds[:-1], bounds[1:]):
        pool.encode(to_dev(ks[:, a:b]), to_dev(vs[:, a:b]), a)
    cont.encode(to_dev(ks), to_dev(vs), 0)
    torch.cuda.synchronize()
    names = ("k_codes", "k_norms", "v_codes", "v_norms")
    for s in range(batch):
        for h in range(cfg.n_kv_heads):
            ref = OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h).packed(n_tiles)
            for name, e in zip(names, ref):
                got = np.stack([_pool_tile(getattr(pool, name), h, table[s, j]) for j in range(n_tiles)])
                assert np.array_equal(got.view(e.dtype), e), (name, s, h)
    # decode: ragged lengths, the same tokens in both layouts
    seq_lens = np.array([seq_len, 130, 1][:batch], np.int32)
    q = np.stack([synth.query(cfg, seq=s) for s in range(batch)])
    out_p = torch.empty((batch, cfg.n_q_heads, 128), dtype=torch.int16, device=dev())
    out_c = torch.empty_like(out_p)
    ws = torch.empty(plan.workspace_size(batch, seq_len), dtype=torch.uint8, device=dev())
    plan.decode_attn_paged(pool.consts, to_dev(q), pool, to_dev(seq_lens), seq_len, out_p, ws)
    plan.decode_attn(cont.consts, to_dev(q), cont.k_codes, cont.k_norms, cont.v_codes, cont.v_norms, seq_len,
                     to_dev(seq_lens), seq_len, out_c, ws)
    torch.cuda.synchronize()
    got = out_p.cpu().numpy().view(np.float16).astype(np.float64)
    assert np.array_equal(out_p.cpu().numpy(), out_c.cpu().numpy())
    for s in range(batch):
        heads = [OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h)
                 for h in range(cfg.n_kv_heads)]
        kh = np.stack([x.k_hat() for x in heads], axis=1)
        vh = np.stack([x.v_hat() for x in heads], axis=1)
        ref = oracle.decode_attention(q[s], kh, vh, int(seq_lens[s]))
        assert rel_l2(got[s], ref).max() <= TOL


@pytest.mark.parametrize("cid,seq_len,batch", [(5, 2048, 1), (4, 700, 3)])
def test_paged_encode_kv_equals_two_encodes(bg, cid, seq_len, batch):
    """bgtq_encode_kv_paged writes every page exactly as the paged key and value encodes do."""
    import torch
    cfg = synth.small(cid, seq_len=seq_len, batch=batch)
    log("paged encode_kv config %d T=%d batch %d" % (cid, seq_len, batch))
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    n_tiles = (seq_len + 63) // 64
    n_pages = batch * n_tiles + 5
    table = np.random.default_rng(7).permutation(n_pages)[:batch * n_tiles].reshape(batch, n_tiles)
    table = table.astype(np.int32)
    fused, two = bg.PagedCache(plan, n_pages, table), bg.PagedCache(plan, n_pages, table)
    ks = np.stack([synth.keys(cfg, seq=s, count=seq_len) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=seq_len) for s in range(batch)])
    bounds = [0, 3, 64, 700, seq_len] if seq_len > 700 else [0, 3, 64, seq_len]
    for a, b in zip(bounds[:-1], bounds[1:]):
        fused.encode_kv(to_dev(ks[:, a:b]), to_dev(vs[:, a:b]), a)
        two.encode(to_dev(ks[:, a:b]), to_dev(vs[:, a:b]), a)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        assert torch.equal(getattr(fused, name), getattr(two, name)), name
    for s in range(batch):
        for h in range(cfg.n_kv_heads):
            ref = OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h).packed(n_tiles)
            got = np.stack([_pool_tile(fused.v_codes, h, table[s, j]) for j in range(n_tiles)])
            assert np.array_equal(got.view(ref[2].dtype), ref[2]), (s, h)


def test_paged_writer_skips_entries_outside_the_pool(bg):
    """A table entry outside [0, n_pages) makes the encode skip that tile (the pool is unchanged)."""
    import torch
    cfg = synth.small(2, seq_len=128)
    bits = np.full((cfg.n_kv_heads, 64), 2, np.int8)
    plan = bg.Plan(bits, 2, 2, cfg.n_q_heads)
    table = np.array([[1, 7]], np.int32)                   # tile 1 -> page 7, outside a 4-page pool
    pool = bg.PagedCache(plan, 4, table)
    pool.encode(to_dev(synth.keys(cfg, count=128)[None]), to_dev(synth.values(cfg, count=128)[None]), 0)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        arr = getattr(pool, name).cpu().numpy()
        assert np.any(arr[:, 1] != 0), name                # page 1 written
        assert np.all(arr[:, [0, 2, 3]] == 0), name        # nothing else touched


def test_paged_decode_step_equals_contiguous(bg):
    """The fused step on a pool: the appended pages and the output equal the contiguous step's."""
    import torch
    cfg = synth.small(4, seq_len=300, batch=3, append=1)
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    max_pages, n_pages = 6, 20
    table = np.random.default_rng(5).permutation(n_pages)[:3 * max_pages].reshape(3, max_pages).astype(np.int32)
    pool = bg.PagedCache(plan, n_pages, table)
    cont = bg.Cache(plan, 3, 64 * max_pages)
    ks = np.stack([synth.keys(cfg, seq=s, count=301) for s in range(3)])
    vs = np.stack([synth.values(cfg, seq=s, count=301) for s in range(3)])
    pool.encode(to_dev(ks[:, :300]), to_dev(vs[:, :300]), 0)
    cont.encode(to_dev(ks[:, :300]), to_dev(vs[:, :300]), 0)
    pos = np.array([300, 130, 5], np.int32)
    k_new = np.stack([ks[s, pos[s]] for s in range(3)])
    v_new = np.stack([vs[s, pos[s]] for s in range(3)])
    q = np.stack([synth.query(cfg, seq=s) for s in range(3)])
    out_p = torch.empty((3, cfg.n_q_heads, 128), dtype=torch.int16, device=dev())
    out_c = torch.empty_like(out_p)
    ws = torch.empty(plan.workspace_size(3, 301), dtype=torch.uint8, device=dev())
    plan.decode_step_paged(pool.consts, to_dev(q), to_dev(k_new), to_dev(v_new), to_dev(pos), 301, pool, out_p, ws)
    cont.step(to_dev(q), to_dev(k_new), to_dev(v_new), to_dev(pos), 301, out_c, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out_p.cpu().numpy(), out_c.cpu().numpy())
    for name in ("k_codes", "k_norms", "v_codes", "v_norms"):
        pa, ca = getattr(pool, name).cpu().numpy(), getattr(cont, name).cpu().numpy()
        for s in range(3):
            for j in range(5):
                assert np.array_equal(pa[:, table[s, j]], ca[s, :, j]), (name, s, j)


@pytest.mark.parametrize("cid,seq_len,n_sink,n_recent", [(4, 700, 4, 128), (2, 900, 64, 300), (1, 300, 0, 64)])
def test_paged_buffered_decode_equals_contiguous(bg, cid, seq_len, n_sink, n_recent):
    """Paged pool + fp16 sink / recent window: the output equals the contiguous buffered decode's
    bit for bit (two sequences, a shuffled block table; the contiguous buffered decode is checked
    against the oracle in test_gpu_buffer)."""
    import torch
    batch = 2
    cfg = synth.small(cid, seq_len=seq_len, batch=batch)
    log("paged buffered decode config %d T=%d sink %d recent %d" % (cid, seq_len, n_sink, n_recent))
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    n_tiles = (seq_len + 63) // 64
    n_pages = batch * n_tiles + 2
    table = np.random.default_rng(11).permutation(n_pages)[:batch * n_tiles].reshape(batch, n_tiles)
    table = table.astype(np.int32)
    pool = bg.PagedCache(plan, n_pages, table)
    cont = bg.Cache(plan, batch, seq_len)
    ks = np.stack([synth.keys(cfg, seq=s, count=seq_len) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=seq_len) for s in range(batch)])
    pool.encode_kv(to_dev(ks), to_dev(vs), 0)
    cont.encode(to_dev(ks), to_dev(vs), 0)
    buf = bg.Buffer(batch, cfg.n_kv_heads, n_sink, n_recent, device=dev())
    buf.append(to_dev(ks), to_dev(vs), 0)
    seq_lens = np.array([seq_len, seq_len], np.int32)  # the buffers hold the last tokens of both
    q = np.stack([synth.query(cfg, seq=s) for s in range(batch)])
    out_p = torch.empty((batch, cfg.n_q_heads, 128), dtype=torch.int16, device=dev())
    out_c = torch.empty_like(out_p)
    ws = torch.empty(plan.workspace_size(batch, seq_len), dtype=torch.uint8, device=dev())
    plan.decode_attn_paged_buffered(pool.consts, to_dev(q), pool, to_dev(seq_lens), seq_len, buf, out_p, ws)
    plan.decode_attn_buffered(cont.consts, to_dev(q), cont.k_codes, cont.k_norms, cont.v_codes, cont.v_norms, seq_len,
                              to_dev(seq_lens), seq_len, buf, out_c, ws)
    torch.cuda.synchronize()
    assert np.array_equal(out_p.cpu().numpy(), out_c.cpu().numpy())
