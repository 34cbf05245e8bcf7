"""Host-side tests of libbgtq: exported symbols, codebooks and rotations against the
oracle, plan validation and argument checks.  No device work is issued."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bg():
    import decode_attention_bgtq_amd as m
    if not os.path.exists(m.LIB_PATH):
        from decode_attention_bgtq_amd import build
        build.build()
    m.load()
    return m


def _header_functions():
    with open(os.path.join(ROOT, "include", "bgtq.h")) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bgtq_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(bg):
    names = _header_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(bg.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bg.EXPORTED) == names


def test_abi_version(bg):
    assert bg.abi_version() == 4


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_codebook_matches_oracle(bg, b):
    c, t, d = bg.codebook(b)
    oc, ot, od, _ = oracle.lloyd_max(b)
    np.testing.assert_allclose(c, oc, rtol=0, atol=1e-12)
    np.testing.assert_allclose(t, ot, rtol=0, atol=1e-12)
    assert abs(d - od) <= 1e-12
    assert t[len(t) // 2] == 0.0


def _bits(seed, avg):
    e = np.exp(np.random.default_rng(seed).normal(0, 2, (3, 64)))
    return np.stack([oracle.greedy_allocate(r, avg, oracle.distortion_table()) for r in e])


def test_plan_rotations_match_oracle(bg):
    bits = _bits(0, 3)
    plan = bg.Plan(bits, 3, 2, n_q_heads=12, seed=7, layer=5)
    np.testing.assert_array_equal(plan.bits(), bits)
    for h in range(3):
        for w in (1, 2, 3, 4):
            d = 2 * int((bits[h] == w).sum())
            got = plan.rotation(h, 0, w)
            if d == 0:
                assert got is None
                continue
            ref = oracle.rotation_for(7, 5, h, 0, w, d)
            assert got.shape == (d, d)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(got.T @ got, np.eye(d), atol=1e-13)
        rv = plan.rotation(h, 1, 2)
        np.testing.assert_allclose(rv, oracle.rotation_for(7, 5, h, 1, 2, 128), rtol=0, atol=1e-12)
        assert plan.rotation(h, 1, 3) is None


def test_plan_sizes(bg):
    bits = _bits(1, 2)
    plan = bg.Plan(bits, 2, 2, n_q_heads=12)
    s = plan.sizes(batch=2, capacity=130)
    tiles = 3
    assert s.k_codes == 2 * 3 * tiles * 8 * 64 * 4
    assert s.k_norms == 2 * 3 * tiles * 64 * 4 * 2
    assert s.v_codes == 2 * 3 * tiles * 128 * 4 * 4
    assert s.v_norms == 2 * 3 * tiles * 64 * 2
    assert s.consts > 0 and s.consts % 256 == 0


def test_plan_validation(bg):
    bits = _bits(2, 3)
    with pytest.raises(bg.BgtqError) as e:
        bg.Plan(bits, 2, 2, n_q_heads=12)          # rows sum to 192, not 128
    assert e.value.status == bg.EBUDGET
    bad = bits.copy()
    bad[0, 0] = 5
    with pytest.raises(bg.BgtqError) as e:
        bg.Plan(bad, 3, 2, n_q_heads=12)
    assert e.value.status == bg.EBUDGET
    for hq in (27, 10):                            # G = 9 (above 8); not a multiple of the KV heads
        with pytest.raises(bg.BgtqError) as e:
            bg.Plan(bits, 3, 2, n_q_heads=hq)
        assert e.value.status == bg.EINVAL
    bg.Plan(bits, 3, 2, n_q_heads=9).close()       # G = 3 runs on the four-head kernels
    with pytest.raises(bg.BgtqError) as e:
        bg.Plan(bits, 3, 5, n_q_heads=12)
    assert e.value.status == bg.EBUDGET
    assert "k_bits" in bg.load().bgtq_last_error().decode() or True


def test_plan_rejects_unknown_pairing(bg):
    bits = np.ascontiguousarray(_bits(3, 2).astype(np.int8))
    desc = bg._PlanDesc(3, 6, 128, 2, 2, bits.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)), 0, 0, 2)
    h = ctypes.c_void_p()
    assert bg.load().bgtq_plan_create(ctypes.byref(desc), ctypes.byref(h)) == bg.EINVAL
    assert "rope_pairing" in bg.load().bgtq_last_error().decode()
    with pytest.raises(ValueError):
        bg.Plan(_bits(3, 2), 2, 2, n_q_heads=6, pairing="other")
    bg.Plan(_bits(3, 2), 2, 2, n_q_heads=6, pairing="interleaved").close()


def test_paged_calls_reject_bad_arguments_before_launch(bg):
    lib = bg.load()
    plan = bg.Plan(_bits(3, 2), 2, 2, n_q_heads=6)
    h = plan.handle
    pg = bg._Pages(256, 4, 10)
    bad = [bg._Pages(None, 4, 10), bg._Pages(256, 0, 10), bg._Pages(256, 4, 0)]
    assert lib.bgtq_encode_k_paged(h, 256, 256, 1, None, 0, 10, 256, 256, None) == bg.EINVAL
    for b in bad:
        assert lib.bgtq_encode_k_paged(h, 256, 256, 1, ctypes.byref(b), 0, 10, 256, 256, None) == bg.EINVAL
        assert lib.bgtq_encode_v_paged(h, 256, 256, 1, ctypes.byref(b), 0, 10, 256, 256, None) == bg.EINVAL
    assert lib.bgtq_encode_k_paged(h, 256, 256, 1, ctypes.byref(pg), 250, 10, 256, 256, None) == bg.ECAPACITY
    args = [h, 256, 256, 256, 256, 256, 256]
    assert lib.bgtq_decode_attn_paged(*args, None, 256, 1, 100, 0.1, 256, 256, 1 << 30, None) == bg.EINVAL
    assert lib.bgtq_decode_attn_paged(*args, ctypes.byref(pg), 256, 1, 257, 0.1, 256, 256, 1 << 30,
                                      None) == bg.ECAPACITY
    assert lib.bgtq_decode_attn_paged(*args, ctypes.byref(bad[1]), 256, 1, 100, 0.1, 256, 256, 1 << 30,
                                      None) == bg.EINVAL
    # the buffered decode step: the step's checks and the buffer checks, before any launch
    sb = [h, 256, 256, 256, 256, 256, 1, 100, 256, 256, 256, 256, 100, 0.1]
    assert lib.bgtq_decode_step_buffered(*sb, 256, 256, 65, 256, 256, 128, 256, 256, 1 << 30, None) == bg.EINVAL
    assert lib.bgtq_decode_step_buffered(*sb, 256, 256, 4, None, 256, 128, 256, 256, 1 << 30, None) == bg.EINVAL
    assert lib.bgtq_decode_step_buffered(*sb, 264, 256, 4, 256, 256, 128, 256, 256, 1 << 30, None) == bg.EINVAL
    assert lib.bgtq_decode_step_buffered(*sb[:7], 101, *sb[8:], 256, 256, 4, 256, 256, 128, 256, 256, 1 << 30,
                                         None) == bg.ECAPACITY
    # paged with the fp16 buffers: the pool checks and the buffer checks, before any launch
    pb = [256, 256, 4, 256, 256, 128]
    assert lib.bgtq_decode_attn_paged_buffered(*args, None, 256, 1, 100, 0.1, *pb, 256, 256, 1 << 30,
                                               None) == bg.EINVAL
    assert lib.bgtq_decode_attn_paged_buffered(*args, ctypes.byref(pg), 256, 1, 257, 0.1, *pb, 256, 256, 1 << 30,
                                               None) == bg.ECAPACITY
    assert lib.bgtq_decode_attn_paged_buffered(*args, ctypes.byref(pg), 256, 1, 100, 0.1, 256, 256, 65, 256, 256,
                                               128, 256, 256, 1 << 30, None) == bg.EINVAL   # n_sink > 64
    assert lib.bgtq_decode_attn_paged_buffered(*args, ctypes.byref(pg), 256, 1, 100, 0.1, None, 256, 4, 256, 256,
                                               128, 256, 256, 1 << 30, None) == bg.EINVAL   # null sink


def test_device_calls_reject_bad_arguments_before_launch(bg):
    lib = bg.load()
    assert lib.bgtq_energy(None, None, 10, 8, 2, 128, 0, None, None) == bg.EINVAL
    assert lib.bgtq_energy(1, 1, 10, 8, 3, 128, 0, 1, None) == bg.EINVAL      # 8 % 3
    assert lib.bgtq_energy(1, 1, 10, 8, 2, 64, 0, 1, None) == bg.EINVAL       # head_dim
    assert lib.bgtq_energy(1, 1, 10, 8, 2, 128, 2, 1, None) == bg.EINVAL      # pairing
    assert lib.bgtq_allocate_device(1, 2, 64, 5, 1, None) == bg.EBUDGET
    assert lib.bgtq_allocate_device(1, 2, 32, 2, 1, None) == bg.EINVAL
    plan = bg.Plan(_bits(3, 2), 2, 2, n_q_heads=6)
    h = plan.handle
    assert lib.bgtq_encode_k(h, 256, 256, 1, 100, 90, 20, 256, 256, None) == bg.ECAPACITY
    assert lib.bgtq_encode_v(h, 256, 256, 1, 100, -1, 20, 256, 256, None) == bg.ECAPACITY
    assert lib.bgtq_encode_k(h, None, 256, 1, 100, 0, 20, 256, 256, None) == bg.EINVAL
    # the fused key + value encode: every check of the two encodes, before any launch
    kv = [h, 256, 256, 256, 1, 100]
    assert lib.bgtq_encode_kv(*kv, 90, 20, 256, 256, 256, 256, None) == bg.ECAPACITY
    assert lib.bgtq_encode_kv(*kv, -1, 20, 256, 256, 256, 256, None) == bg.ECAPACITY
    assert lib.bgtq_encode_kv(h, 256, 256, None, 1, 100, 0, 20, 256, 256, 256, 256, None) == bg.EINVAL
    assert lib.bgtq_encode_kv(*kv, 0, 20, 256, 256, None, 256, None) == bg.EINVAL
    assert lib.bgtq_encode_kv(h, 256, 256, 264, 1, 100, 0, 20, 256, 256, 256, 256, None) == bg.EINVAL  # align
    assert lib.bgtq_encode_kv(h, 256, 256, 256, 0, 100, 0, 20, 256, 256, 256, 256, None) == bg.EINVAL
    pg = bg._Pages(None, 4, 10)
    assert lib.bgtq_encode_kv_paged(h, 256, 256, 256, 1, ctypes.byref(pg), 0, 10, 256, 256, 256, 256,
                                    None) == bg.EINVAL
    assert lib.bgtq_encode_kv_paged(h, 256, 256, 256, 1, None, 0, 10, 256, 256, 256, 256, None) == bg.EINVAL
    args = [h, 256, 256, 256, 256, 256, 256]
    assert lib.bgtq_decode_attn(*args, 100, 256, 1, 101, 0.1, 256, 256, 1 << 30, None) == bg.ECAPACITY
    assert lib.bgtq_decode_attn(*args, 100, 256, 1, 0, 0.1, 256, 256, 1 << 30, None) == bg.ECAPACITY
    assert lib.bgtq_decode_attn(*args, 1 << 32, 256, 1, 1 << 31, 0.1, 256, 256, 1 << 30, None) == bg.EINVAL
    assert lib.bgtq_decode_attn(*args, 100, 256, 1, 50, 0.1, 256, 256, 16, None) == bg.EWORKSPACE
    assert lib.bgtq_decode_attn(*args, 100, 256, 1, 50, -1.0, 256, 256, 1 << 30, None) == bg.EINVAL
    assert lib.bgtq_decode_attn(h, 256, None, 256, 256, 256, 256, 100, 256, 1, 50, 0.1, 256, 256, 1 << 30,
                                None) == bg.EINVAL
    assert lib.bgtq_plan_upload(h, 255, None) == bg.EINVAL                  # misaligned
    assert lib.bgtq_codebook(0, None, None, None) == bg.EINVAL


@pytest.mark.parametrize("avg", [0, 1, 2, 3, 4])
def test_host_allocation_matches_oracle_greedy(bg, avg):
    """bgtq_allocate (host, synchronous) gives the oracle's greedy widths bit for bit: random
    log-normal energies, a row of equal energies (uniform widths), a row with zero-energy
    blocks and a row of pairwise-equal energies (ties to the lowest block)."""
    rng = np.random.default_rng(100 + avg)
    e = np.exp(rng.normal(0, 2, (6, 64)))
    e[1] = 1.0
    e[2, :20] = 0.0
    e[3] = np.repeat(np.exp(rng.normal(0, 1, 32)), 2)
    e[4] = np.exp(rng.normal(0, 8, 64))                 # a wide range of scales
    got = bg.allocate(e, avg)
    dist = oracle.distortion_table()
    ref = np.stack([oracle.greedy_allocate(r, avg, dist) for r in e])
    np.testing.assert_array_equal(got, ref)
    assert np.all(got[1] == avg) and np.all(got.sum(1) == 64 * avg)


def test_host_allocation_rejects_bad_energies(bg):
    lib = bg.load()
    bits = np.full((2, 64), 7, np.int8)
    for bad in (-1.0, np.nan, np.inf):
        e = np.ones((2, 64))
        e[1, 5] = bad
        assert lib.bgtq_allocate(e.ctypes.data, 2, 64, 2, bits.ctypes.data) == bg.EINVAL
        assert "finite" in lib.bgtq_last_error().decode()
    assert np.all(bits == 7)                             # nothing written on an error
    e = np.ones((2, 64))
    assert lib.bgtq_allocate(e.ctypes.data, 2, 64, 5, bits.ctypes.data) == bg.EBUDGET
    assert lib.bgtq_allocate(e.ctypes.data, 2, 32, 2, bits.ctypes.data) == bg.EINVAL
    assert lib.bgtq_allocate(None, 2, 64, 2, bits.ctypes.data) == bg.EINVAL


def test_binding_rejects_bad_tensors_before_the_call(bg):
    """The binding checks layout, element type, shape and device before an address crosses the
    ABI: a strided time slice, a wrong head count, a wrong dtype or a host tensor raise."""
    import torch
    plan = bg.Plan(_bits(3, 2), 2, 2, n_q_heads=6)
    k = torch.zeros((2, 40, 3, 128), dtype=torch.float16)
    codes = torch.zeros(16, dtype=torch.int32)
    norms = torch.zeros(16, dtype=torch.int16)
    with pytest.raises(ValueError, match="contiguous"):
        plan.encode_k(codes, k[:, 5:20], 64, 0, codes, norms)
    with pytest.raises(ValueError, match="shape"):
        plan.encode_k(codes, torch.zeros((2, 40, 4, 128), dtype=torch.float16), 64, 0, codes, norms)
    with pytest.raises(ValueError, match="2-byte"):
        plan.encode_v(codes, k.float(), 64, 0, codes, norms)
    with pytest.raises(ValueError, match="GPU"):
        plan.encode_k(codes, k, 64, 0, codes, norms)
    q = torch.zeros((2, 6, 128), dtype=torch.float16)
    out = torch.zeros((2, 6, 128), dtype=torch.float16)
    ws = torch.zeros(64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="int32"):
        plan.decode_attn(codes, q, codes, norms, codes, norms, 64, torch.zeros(2, dtype=torch.int64), 64, out, ws)
    with pytest.raises(ValueError, match="shape"):
        plan.decode_attn(codes, q, codes, norms, codes, norms, 64, torch.zeros(3, dtype=torch.int32), 64, out, ws)
    with pytest.raises(ValueError, match="shape"):
        plan.decode_attn(codes, torch.zeros((2, 4, 128), dtype=torch.float16), codes, norms, codes, norms, 64,
                         torch.zeros(2, dtype=torch.int32), 64, out, ws)
    with pytest.raises(ValueError, match="GPU"):
        plan.decode_attn(codes, q, codes, norms, codes, norms, 64, torch.zeros(2, dtype=torch.int32), 64, out, ws)
    with pytest.raises(ValueError, match="shape"):
        bg.allocate_device(torch.zeros((3, 32), dtype=torch.float64), 2, torch.zeros((3, 32), dtype=torch.int8))
