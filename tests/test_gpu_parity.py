"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Energies, allocations, packed codes and fp16 norms must be bit-exact; decode
outputs must be within 2e-3 relative L2 per (sequence, query head) (fp16 I/O,
fp32 accumulation).
"""
import math

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


def _energy_alloc(bg, q_cal, k_cal, n_kv, avg, pairing="half"):
    import torch
    e = torch.empty((n_kv, 64), dtype=torch.float64, device="cuda")
    bg.energy(to_dev(q_cal), to_dev(k_cal), n_kv, e, pairing=pairing)
    bits = torch.empty((n_kv, 64), dtype=torch.int8, device="cuda")
    bg.allocate_device(e, avg, bits)
    torch.cuda.synchronize()
    e_host, b_dev = e.cpu().numpy(), bits.cpu().numpy()
    assert np.array_equal(bg.allocate(e_host, avg), b_dev)      # host greedy = device kernel
    return e_host, b_dev


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_energy_and_allocation_bitexact(bg, cid):
    cfg = synth.CONFIGS[cid]
    log("config %d: calibration %d tokens" % (cid, cfg.n_cal))
    q_cal, k_cal = synth.calibration(cfg)
    e_gpu, b_gpu = _energy_alloc(bg, q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    e_ref, b_ref = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    assert np.array_equal(e_gpu, e_ref)
    assert np.array_equal(b_gpu, b_ref)
    assert np.all(b_gpu.sum(1) == 64 * cfg.k_bits)


@pytest.mark.parametrize("cid", [1, 3])
def test_energy_and_allocation_bitexact_interleaved(bg, cid):
    cfg = synth.small(cid, pairing="interleaved")
    log("config %d interleaved: calibration %d tokens" % (cid, cfg.n_cal))
    q_cal, k_cal = synth.calibration(cfg)
    e_gpu, b_gpu = _energy_alloc(bg, q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits, "interleaved")
    e_ref, b_ref = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits, "interleaved")
    assert np.array_equal(e_gpu, e_ref)
    assert np.array_equal(b_gpu, b_ref)
    # the interleaved twin of a half-split config sees the same blocks
    qh, kh = synth.calibration(synth.CONFIGS[cid])
    e_half, _ = _energy_alloc(bg, qh, kh, cfg.n_kv_heads, cfg.k_bits)
    assert np.array_equal(e_gpu, e_half)


def test_allocation_budgets_and_uniform(bg):
    import torch
    rng = np.random.default_rng(9)
    e = np.exp(rng.normal(0, 2, (5, 64)))
    e[1] = 1.0                                     # equal energies: uniform widths
    e[2, :10] = 0.0                                # zero-energy blocks
    dist = oracle.distortion_table()
    for avg in range(5):
        ed = torch.from_numpy(e).cuda()
        bits = torch.empty((5, 64), dtype=torch.int8, device="cuda")
        bg.allocate_device(ed, avg, bits)
        torch.cuda.synchronize()
        got = bits.cpu().numpy()
        ref = np.stack([oracle.greedy_allocate(e[h], avg, dist) for h in range(5)])
        assert np.array_equal(got, ref), avg
        assert np.array_equal(bg.allocate(e, avg), ref), avg
        assert np.all(got[1] == avg)


def _encode_case(bg, cfg, seq_len, batch=1, capacity=None, bits=None, chunks=None, fused=False):
    """Encode `seq_len` tokens per sequence on the GPU (optionally in several appends; with
    `fused`, keys and values in one bgtq_encode_kv call) and compare every packed array with
    the oracle's."""
    import torch
    capacity = capacity or seq_len
    if bits is None:
        q_cal, k_cal = synth.calibration(cfg)
        _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits, cfg.pairing)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed, layer=0, pairing=cfg.pairing)
    cache = bg.Cache(plan, batch, capacity, device="cuda")
    ks = np.stack([synth.keys(cfg, seq=s, count=seq_len) for s in range(batch)])
    vs = np.stack([synth.values(cfg, seq=s, count=seq_len) for s in range(batch)])
    bounds = chunks or [0, seq_len]
    for a, b in zip(bounds[:-1], bounds[1:]):
        if fused:
            cache.encode_kv(to_dev(ks[:, a:b]), to_dev(vs[:, a:b]), a)
        else:
            cache.encode(to_dev(ks[:, a:b]), to_dev(vs[:, a:b]), a)
    torch.cuda.synchronize()
    heads = {}
    for s in range(batch):
        for h in range(cfg.n_kv_heads):
            ref = OracleHead(ks[s, :, h], vs[s, :, h], bits[h], cfg.v_bits, cfg.seed, 0, h, cfg.pairing)
            got = gpu_arrays(cache, s, h)
            exp = ref.packed(cache.tiles)
            for name, g, e in zip(("k_codes", "k_norms", "v_codes", "v_norms"), got, exp):
                if not np.array_equal(g, e):
                    bad = np.argwhere(g != e)
                    raise AssertionError("%s mismatch seq %d head %d at %s (of %d)" %
                                         (name, s, h, bad[:5].tolist(), len(bad)))
            heads[(s, h)] = ref
    return plan, cache, bits, ks, vs, heads


@pytest.mark.parametrize("cid,seq_len", [(1, 4096), (1, 1), (1, 63), (1, 65), (2, 1000), (3, 700), (5, 130)])
def test_encode_bitexact(bg, cid, seq_len):
    log("encode config %d T=%d" % (cid, seq_len))
    _encode_case(bg, synth.small(cid, seq_len=seq_len), seq_len)


def test_encode_batched_and_appended(bg):
    cfg = synth.small(4, seq_len=300, batch=3)
    log("encode batch 3, appends at 0/37/64/101/200")
    _encode_case(bg, cfg, 300, batch=3, capacity=320, chunks=[0, 37, 64, 101, 200, 300])


# bgtq_encode_kv: one launch for keys and values where the two encodes fill at most one round
# of compute units (half tiles below half a round), else the two encodes in turn; every case
# bit-exact against the oracle.  (3, 3000): 47 tiles x 8 heads takes the two-launch path;
# the chunked batch mixes appends of 5, 27, 37 and 199 tokens (the few-token path at 5).
@pytest.mark.parametrize("cid,seq_len,batch,chunks", [
    (5, 4096, 1, None), (3, 700, 1, None), (2, 1000, 1, None), (1, 63, 1, None), (3, 3000, 1, None),
    (4, 300, 3, [0, 5, 32, 69, 101, 300])])
def test_encode_kv_bitexact(bg, cid, seq_len, batch, chunks):
    log("encode_kv config %d T=%d batch %d" % (cid, seq_len, batch))
    cfg = synth.small(cid, seq_len=seq_len, batch=batch)
    _encode_case(bg, cfg, seq_len, batch=batch, capacity=seq_len + 20, chunks=chunks, fused=True)


def test_encode_kv_append_at_offset(bg):
    """A 4096-token append at position 8192 behind a prefill (the long-context workload's
    append, reduced), keys and values in one call."""
    cfg = synth.small(5, seq_len=8192 + 4096)
    log("encode_kv append of 4096 at 8192")
    _encode_case(bg, cfg, 8192 + 4096, capacity=8192 + 4096 + 64, chunks=[0, 8192, 8192 + 4096], fused=True)


def test_encode_zero_and_uniform(bg):
    import torch
    cfg = synth.small(2, seq_len=64)
    bits = np.full((cfg.n_kv_heads, 64), 3, np.int8)          # uniform TQ-MSE special case
    plan = bg.Plan(bits, 3, 3, cfg.n_q_heads)
    cache = bg.Cache(plan, 1, 64, device="cuda")
    k = synth.keys(cfg, count=64)
    k[5] = 0
    v = synth.values(cfg, count=64)
    v[7] = 0
    cache.encode(to_dev(k[None]), to_dev(v[None]), 0)
    torch.cuda.synchronize()
    for h in range(cfg.n_kv_heads):
        ref = OracleHead(k[:, h], v[:, h], bits[h], 3, 0, 0, h)
        for g, e in zip(gpu_arrays(cache, 0, h), ref.packed(1)):
            assert np.array_equal(g, e)


def test_rotate_queries(bg):
    import torch
    cfg = synth.small(3, seq_len=64, batch=2)
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads)
    cache = bg.Cache(plan, 2, 64, device="cuda")
    q = np.stack([synth.query(cfg, seq=s) for s in range(2)])
    qr = torch.empty((2, cfg.n_q_heads, 128), dtype=torch.float32, device="cuda")
    plan.rotate_queries(cache.consts, to_dev(q), qr)
    torch.cuda.synchronize()
    got = qr.cpu().numpy()
    for s in range(2):
        for h in range(cfg.n_q_heads):
            kvh = h // cfg.group
            ref = np.zeros(128)
            off = 0
            for w, coords in oracle.groups_for(bits[kvh]):
                pi = oracle.rotation_for(0, 0, kvh, 0, w, coords.size)
                ref[off:off + coords.size] = pi @ q[s, h, coords].astype(np.float64)
                off += coords.size
            np.testing.assert_allclose(got[s, h], ref, rtol=0, atol=2e-6 * np.abs(ref).max())


def _decode_check(bg, cfg, seq_len, batch=1, seq_lens=None, capacity=None):
    seq_lens = list(seq_lens) if seq_lens is not None else [seq_len] * batch
    plan, cache, bits, ks, vs, heads = _encode_case(bg, cfg, seq_len, batch=batch, capacity=capacity)
    q = np.stack([synth.query(cfg, seq=s) for s in range(batch)])
    got = decode_gpu(plan, cache, q, seq_lens, max(max(seq_lens), 1))
    worst = 0.0
    for s in range(batch):
        kh = np.stack([heads[(s, h)].k_hat() for h in range(cfg.n_kv_heads)], axis=1)
        vh = np.stack([heads[(s, h)].v_hat() for h in range(cfg.n_kv_heads)], axis=1)
        ref = oracle.decode_attention(q[s], kh, vh, seq_lens[s])
        if seq_lens[s] == 0:
            assert np.all(got[s] == 0.0)
            continue
        r = rel_l2(got[s], ref)
        worst = max(worst, float(r.max()))
        assert r.max() <= TOL, (s, r.max())
    log("decode worst rel-L2 %.3e" % worst)
    return plan, cache, q, got


@pytest.mark.parametrize("cid,seq_len", [(1, 4096), (1, 1), (1, 100), (2, 2000), (3, 3000), (5, 1500)])
def test_decode_matches_oracle(bg, cid, seq_len):
    log("decode config %d T=%d" % (cid, seq_len))
    _decode_check(bg, synth.small(cid, seq_len=seq_len), seq_len)


@pytest.mark.parametrize("cid,seq_len", [(1, 1000), (3, 3000), (4, 777)])
def test_decode_interleaved_pairing(bg, cid, seq_len):
    """Interleaved RoPE pairing end to end: the plan's key groups take coordinates (2j, 2j+1)."""
    log("decode config %d interleaved T=%d" % (cid, seq_len))
    _decode_check(bg, synth.small(cid, seq_len=seq_len, batch=2 if cid == 4 else None,
                                  pairing="interleaved"), seq_len, batch=2 if cid == 4 else 1)


def test_decode_ragged_batch_and_empty(bg):
    cfg = synth.small(4, seq_len=1100, batch=5)
    _decode_check(bg, cfg, 1100, batch=5, seq_lens=[0, 1, 64, 700, 1100], capacity=1152)


@pytest.mark.parametrize("g,vb", [(1, 1), (2, 2), (4, 3), (8, 4), (8, 1), (4, 4), (2, 3), (1, 2),
                                  (3, 2), (5, 3), (6, 1), (7, 2), (7, 4)])  # 3, 5..7: padded kernels
def test_decode_group_and_value_widths(bg, g, vb):
    cfg = synth.small(2, seq_len=777, n_kv_heads=2, n_q_heads=2 * g, v_bits=vb, k_bits=2)
    _decode_check(bg, cfg, 777)


@pytest.mark.parametrize("g,kb,vb", [(8, 4, 3), (8, 3, 4), (6, 4, 4), (4, 4, 3), (8, 3, 3)])
def test_decode_wide_tiles(bg, g, kb, vb):
    """Key and value widths whose tiles decide the occupancy: eight heads at K4V3, K3V4 and K4V4
    (two waves per SIMD, query operands in registers), four heads at K4V3 (three waves per SIMD,
    12-wave workgroups), eight heads at K3V3 (three waves, query operands in LDS)."""
    cfg = synth.small(2, seq_len=1500, n_kv_heads=2, n_q_heads=2 * g, v_bits=vb, k_bits=kb)
    _decode_check(bg, cfg, 1500)


def test_decode_zero_bit_keys(bg):
    """avg 0 bits for keys: every logit is 0, attention is the mean of the values."""
    cfg = synth.small(2, seq_len=200, k_bits=0)
    bits = np.zeros((cfg.n_kv_heads, 64), np.int8)
    plan, cache, _, ks, vs, heads = _encode_case(bg, cfg, 200, bits=bits)
    q = synth.query(cfg)[None]
    got = decode_gpu(plan, cache, q, [200], 200)
    for h in range(cfg.n_q_heads):
        ref = heads[(0, h // cfg.group)].v_hat().mean(0)
        assert rel_l2(got[0, h], ref) <= TOL


def test_encode_kv_zero_bit_keys(bg):
    """bgtq_encode_kv with a zero-bit key plan: no key words, zero key norms, the values
    bit-exact, and the decode the mean of the values."""
    cfg = synth.small(2, seq_len=200, k_bits=0)
    bits = np.zeros((cfg.n_kv_heads, 64), np.int8)
    plan, cache, _, ks, vs, heads = _encode_case(bg, cfg, 200, bits=bits, fused=True)
    q = synth.query(cfg)[None]
    got = decode_gpu(plan, cache, q, [200], 200)
    for h in range(cfg.n_q_heads):
        ref = heads[(0, h // cfg.group)].v_hat().mean(0)
        assert rel_l2(got[0, h], ref) <= TOL


def test_decode_deterministic(bg):
    cfg = synth.small(3, seq_len=5000)
    plan, cache, q, got = _decode_check(bg, cfg, 5000)
    again = decode_gpu(plan, cache, q, [5000], 5000)
    assert np.array_equal(got, again)


def test_decode_custom_scale(bg):
    cfg = synth.small(1, seq_len=500)
    plan, cache, bits, ks, vs, heads = _encode_case(bg, cfg, 500)
    q = synth.query(cfg)[None]
    got = decode_gpu(plan, cache, q, [500], 500, scale=0.05)
    ref = oracle.decode_attention(q[0], heads[(0, 0)].k_hat()[:, None], heads[(0, 0)].v_hat()[:, None], 500,
                                  scale=0.05)
    assert rel_l2(got[0], ref).max() <= TOL


def test_full_size_128k_sampled(bg):
    """The 128K Llama-3.1-8B-shaped layer at full size in the benchmark's launch configuration:
    all codes of two KV heads and sampled tiles of the rest are bit-exact, and the decode
    output of the query heads of those two KV heads matches the oracle."""
    import torch
    cfg = synth.CONFIGS[3]
    t = cfg.seq_len
    log("128K: calibration + allocation")
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = _energy_alloc(bg, q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    cache = bg.Cache(plan, 1, t, device="cuda")
    log("128K: generate + encode")
    k = synth.keys(cfg, count=t)
    v = synth.values(cfg, count=t)
    cache.encode(to_dev(k[None]), to_dev(v[None]), 0)
    q = synth.query(cfg)[None]
    got = decode_gpu(plan, cache, q, [t], t)
    log("128K: buffered decode (4 sink + 128 recent fp16 tokens)")
    buf = bg.Buffer(1, cfg.n_kv_heads, 4, 128)
    buf.append(to_dev(k[None]), to_dev(v[None]), 0)
    got_buf = decode_gpu(plan, cache, q, [t], t, buf=buf)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for h in range(cfg.n_kv_heads):
        full = h in (0, 5)
        if full:
            idx = np.arange(t)
        else:
            tiles = rng.choice(t // 64, 8, replace=False)
            idx = (tiles[:, None] * 64 + np.arange(64)[None]).reshape(-1)
        log("128K: oracle head %d (%s)" % (h, "full" if full else "8 tiles"))
        ref = OracleHead(k[idx, h], v[idx, h], bits[h], cfg.v_bits, cfg.seed, 0, h)
        kc, kn, vc, vn = gpu_arrays(cache, 0, h)
        from oracle import layout
        gk_codes, gk_norms = layout.unpack_k(kc, kn, bits[h], t)
        gv_codes, gv_norms = layout.unpack_v(vc, vn, cfg.v_bits, t)
        assert np.array_equal(gk_codes[idx], ref.kc) and np.array_equal(gk_norms[idx], ref.kn)
        assert np.array_equal(gv_codes[idx], ref.vc) and np.array_equal(gv_norms[idx], ref.vn)
        if full:
            o = np.stack([oracle.softmax_attention(q[0, hh].astype(np.float64), ref.k_hat(), ref.v_hat(),
                                                   1 / math.sqrt(128))
                          for hh in range(h * cfg.group, (h + 1) * cfg.group)])
            r = rel_l2(got[0, h * cfg.group:(h + 1) * cfg.group], o)
            log("128K: head %d rel-L2 max %.3e" % (h, r.max()))
            assert r.max() <= TOL
            ob = oracle.decode_attention_buffered(q[0, h * cfg.group:(h + 1) * cfg.group], k[:, h:h + 1],
                                                  v[:, h:h + 1], ref.k_hat()[:, None], ref.v_hat()[:, None],
                                                  t, 4, 128)
            rb = rel_l2(got_buf[0, h * cfg.group:(h + 1) * cfg.group], ob)
            log("128K: head %d buffered rel-L2 max %.3e" % (h, rb.max()))
            assert rb.max() <= TOL


def test_decode_invariant_to_split_count(bg):
    """The same cache and query decoded with different max_seq_len bounds (so different split
    counts, visible as different workspace sizes) agree to fp16 output rounding."""
    cfg = synth.small(2, seq_len=3000)
    plan, cache, bits, ks, vs, heads = _encode_case(bg, cfg, 3000, capacity=65536)
    q = synth.query(cfg)[None]
    outs, sizes = [], []
    for msl in (3000, 9000, 65536):
        sizes.append(plan.workspace_size(1, msl))
        outs.append(decode_gpu(plan, cache, q, [3000], msl))
    assert len(set(sizes)) == 3
    for o in outs[1:]:
        r = rel_l2(o[0], outs[0][0])
        assert r.max() <= 1e-3, r.max()      # one fp16 ulp is ~1e-3 relative
    ref = oracle.decode_attention(q[0], np.stack([heads[(0, h)].k_hat() for h in range(2)], axis=1),
                                  np.stack([heads[(0, h)].v_hat() for h in range(2)], axis=1), 3000)
    for o in outs:
        assert rel_l2(o[0], ref).max() <= TOL


def test_decode_on_two_streams_shares_the_plan(bg):
    """One plan and constant image used by decode calls on two streams at once (separate
    workspaces and outputs) gives the same outputs as the calls one after the other."""
    import torch
    cfg = synth.small(3, seq_len=2000)
    plan, cache, bits, ks, vs, heads = _encode_case(bg, cfg, 2000)
    q = to_dev(synth.query(cfg)[None])
    lens = to_dev(np.array([2000], np.int32))
    serial = decode_gpu(plan, cache, synth.query(cfg)[None], [2000], 2000)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((1, cfg.n_q_heads, 128), dtype=torch.int16, device="cuda") for _ in streams]
    wss = [torch.empty(plan.workspace_size(1, 2000), dtype=torch.uint8, device="cuda") for _ in streams]
    torch.cuda.synchronize()
    for _ in range(3):
        for st, o, ws in zip(streams, outs, wss):
            with torch.cuda.stream(st):
                plan.decode_attn(cache.consts, q, cache.k_codes, cache.k_norms, cache.v_codes, cache.v_norms,
                                 cache.capacity, lens, 2000, o, ws, stream=st)
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(o.cpu().numpy().view(np.float16).astype(np.float64), serial)


def test_full_size_512k_with_append_sampled(bg):
    """The 512K Qwen2.5-3B-shaped layer at full size, then its 4096-token append at position
    524,288: sampled tiles (the appended ones included) bit-exact, and the decode over all
    528,384 tokens of KV head 0's query heads within tolerance of the oracle."""
    import torch
    cfg = synth.CONFIGS[5]
    t, app = cfg.seq_len, cfg.append
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = _energy_alloc(bg, q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    cache = bg.Cache(plan, 1, t + app, device="cuda")
    log("512K: generate + encode + append")
    k = synth.keys(cfg, count=t + app)
    v = synth.values(cfg, count=t + app)
    cache.encode(to_dev(k[None, :t]), to_dev(v[None, :t]), 0)
    cache.encode(to_dev(k[None, t:]), to_dev(v[None, t:]), t)
    q = synth.query(cfg, pos=t + app)[None]
    got = decode_gpu(plan, cache, q, [t + app], t + app)
    torch.cuda.synchronize()
    from oracle import layout
    rng = np.random.default_rng(1)
    for h in range(cfg.n_kv_heads):
        full = h == 0
        if full:
            idx = np.arange(t + app)
        else:
            tiles = np.concatenate([rng.choice(t // 64, 6, replace=False), [t // 64, (t + app) // 64 - 1]])
            idx = (tiles[:, None] * 64 + np.arange(64)[None]).reshape(-1)
        log("512K: oracle head %d (%s)" % (h, "full" if full else "8 tiles"))
        ref = OracleHead(k[idx, h], v[idx, h], bits[h], cfg.v_bits, cfg.seed, 0, h)
        kc, kn, vc, vn = gpu_arrays(cache, 0, h)
        gk_codes, gk_norms = layout.unpack_k(kc, kn, bits[h], t + app)
        gv_codes, gv_norms = layout.unpack_v(vc, vn, cfg.v_bits, t + app)
        assert np.array_equal(gk_codes[idx], ref.kc) and np.array_equal(gk_norms[idx], ref.kn)
        assert np.array_equal(gv_codes[idx], ref.vc) and np.array_equal(gv_norms[idx], ref.vn)
        if full:
            o = np.stack([oracle.softmax_attention(q[0, hh].astype(np.float64), ref.k_hat(), ref.v_hat(),
                                                   1 / math.sqrt(128))
                          for hh in range(cfg.group)])
            r = rel_l2(got[0, :cfg.group], o)
            log("512K: head 0 rel-L2 max %.3e" % r.max())
            assert r.max() <= TOL


def test_full_size_16x32k_sampled(bg):
    """The batched 16 x 32K Llama-3.1-8B-shaped layer at full size: sampled tiles of every
    sequence bit-exact, and the decode of sequences 0 and 15 (query heads of KV head 3) within
    tolerance of the oracle over all 32,768 tokens."""
    import torch
    cfg = synth.CONFIGS[4]
    t, nb = cfg.seq_len, cfg.batch
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = _energy_alloc(bg, q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    cache = bg.Cache(plan, nb, t, device="cuda")
    log("16x32K: generate + encode")
    ks = np.stack([synth.keys(cfg, seq=s, count=t) for s in range(nb)])
    vs = np.stack([synth.values(cfg, seq=s, count=t) for s in range(nb)])
    cache.encode(to_dev(ks), to_dev(vs), 0)
    q = np.stack([synth.query(cfg, seq=s) for s in range(nb)])
    got = decode_gpu(plan, cache, q, [t] * nb, t)
    torch.cuda.synchronize()
    from oracle import layout
    rng = np.random.default_rng(2)
    h = 3
    for s in range(nb):
        full = s in (0, nb - 1)
        idx = np.arange(t) if full else (rng.choice(t // 64, 2, replace=False)[:, None] * 64
                                         + np.arange(64)[None]).reshape(-1)
        ref = OracleHead(ks[s, idx, h], vs[s, idx, h], bits[h], cfg.v_bits, cfg.seed, 0, h)
        kc, kn, vc, vn = gpu_arrays(cache, s, h)
        gk_codes, gk_norms = layout.unpack_k(kc, kn, bits[h], t)
        gv_codes, gv_norms = layout.unpack_v(vc, vn, cfg.v_bits, t)
        assert np.array_equal(gk_codes[idx], ref.kc) and np.array_equal(gk_norms[idx], ref.kn)
        assert np.array_equal(gv_codes[idx], ref.vc) and np.array_equal(gv_norms[idx], ref.vn)
        if full:
            o = np.stack([oracle.softmax_attention(q[s, hh].astype(np.float64), ref.k_hat(), ref.v_hat(),
                                                   1 / math.sqrt(128))
                          for hh in range(h * cfg.group, (h + 1) * cfg.group)])
            r = rel_l2(got[s, h * cfg.group:(h + 1) * cfg.group], o)
            log("16x32K: sequence %d rel-L2 max %.3e" % (s, r.max()))
            assert r.max() <= TOL


@pytest.mark.parametrize("cid,vscale", [(3, 300.0), (2, 300.0), (3, 1e-3), (1, 3000.0)])
def test_decode_value_norm_range(bg, cid, vscale):
    """Value norms far from the synthetic ~11 (x300: ~3.4e3; x3000: ~3.4e4, near the top of fp16;
    x1e-3: ~0.011) with keys whose scale grows along the sequence, so that the logits keep
    rising and the running maximum is overtaken again and again.  The softmax-weight x
    value-norm operand must stay finite and accurate: outputs within tolerance of the oracle."""
    import torch
    t = 3000
    cfg = synth.small(cid, seq_len=t)
    q_cal, k_cal = synth.calibration(cfg)
    _, bits = ref_bits(q_cal, k_cal, cfg.n_kv_heads, cfg.k_bits)
    plan = bg.Plan(bits, cfg.k_bits, cfg.v_bits, cfg.n_q_heads, seed=cfg.seed)
    cache = bg.Cache(plan, 1, t, device="cuda")
    ramp = np.linspace(0.25, 3.0, t)[:, None, None]
    k = (synth.keys(cfg, count=t).astype(np.float64) * ramp).astype(np.float16)
    v = (synth.values(cfg, count=t).astype(np.float64) * vscale).astype(np.float16)
    assert np.all(np.isfinite(k)) and np.all(np.isfinite(v))
    log("value norm range: config %d, value scale %g (norms up to %.3g)" %
        (cid, vscale, float(np.linalg.norm(v.astype(np.float64), axis=-1).max())))
    cache.encode(to_dev(k[None]), to_dev(v[None]), 0)
    torch.cuda.synchronize()
    q = synth.query(cfg)[None]
    got = decode_gpu(plan, cache, q, [t], t)
    assert np.all(np.isfinite(got))
    kh = np.stack([OracleHead(k[:, h], v[:, h], bits[h], cfg.v_bits, cfg.seed, 0, h).k_hat()
                   for h in range(cfg.n_kv_heads)], axis=1)
    vh = np.stack([OracleHead(k[:, h], v[:, h], bits[h], cfg.v_bits, cfg.seed, 0, h).v_hat()
                   for h in range(cfg.n_kv_heads)], axis=1)
    ref = oracle.decode_attention(q[0], kh, vh, t)
    r = rel_l2(got[0], ref)
    log("value norm range: worst rel-L2 %.3e" % r.max())
    assert r.max() <= TOL
