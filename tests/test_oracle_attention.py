"""Pins of the oracle's attention and of the RoPE block decomposition."""
import math

import numpy as np
from scipy import special

import oracle
import synth


def test_rope_block_decomposition_identity():
    """Sum of per-block logits equals the RoPE'd dot product (the pages' decomposition).

    At positions below 4096 the two sides agree to 1e-12 * |q||k|.  At large
    positions the float64 angles p * omega_j carry an absolute rounding error
    of about p * 2^-52, so the bound grows with the position.
    """
    rng = np.random.default_rng(0)
    for trial in range(100):
        q, k = rng.normal(0, 3, 128), rng.normal(0, 3, 128)
        hi = 4096 if trial < 50 else 600000
        m, n = rng.integers(0, hi, 2)
        theta = float(rng.choice([1e4, 5e5, 1e6]))
        blocks = oracle.block_logits(q, k, float(m), float(n), theta)
        full = oracle.rope_blocks(q, float(m), theta) @ oracle.rope_blocks(k, float(n), theta)
        scale = max(1.0, np.linalg.norm(q) * np.linalg.norm(k))
        tol = 1e-12 if hi == 4096 else 1e-12 + 8 * 2.0 ** -52 * max(m, n)
        assert abs(blocks.sum() - full) <= tol * scale


def test_interleaved_rope_is_complex_multiplication():
    """Interleaved RoPE multiplies z_j = x[2j] + i x[2j+1] by exp(i p omega_j); the sum of the
    interleaved block logits equals the dot product of the rotated vectors."""
    rng = np.random.default_rng(2)
    for trial in range(40):
        x = rng.normal(0, 2, 128)
        p = float(rng.integers(0, 5000))
        theta = float(rng.choice([1e4, 5e5]))
        z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * p * theta ** (-np.arange(64) / 64.0))
        got = oracle.rope_blocks(x, p, theta, "interleaved")
        np.testing.assert_allclose(got[0::2], z.real, atol=1e-11)
        np.testing.assert_allclose(got[1::2], z.imag, atol=1e-11)
        q, k = rng.normal(0, 3, 128), rng.normal(0, 3, 128)
        m, n = rng.integers(0, 4096, 2)
        blocks = oracle.block_logits(q, k, float(m), float(n), theta, "interleaved")
        full = oracle.rope_blocks(q, float(m), theta, "interleaved") @ oracle.rope_blocks(k, float(n), theta,
                                                                                          "interleaved")
        assert abs(blocks.sum() - full) <= 1e-12 * max(1.0, np.linalg.norm(q) * np.linalg.norm(k))


def test_generator_rope_matches_oracle_rope():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1, (5, 1, 128))
    pos = np.array([0, 1, 77, 4095, 524287])
    got = synth.rope_f64(x, pos, 5e5)
    for i, p in enumerate(pos):
        np.testing.assert_allclose(got[i, 0], oracle.rope_blocks(x[i, 0], float(p), 5e5), atol=1e-12)
    got = synth.rope_f64(x, pos, 5e5, "interleaved")
    for i, p in enumerate(pos):
        np.testing.assert_allclose(got[i, 0], oracle.rope_blocks(x[i, 0], float(p), 5e5, "interleaved"),
                                   atol=1e-12)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(2)
    k, v = rng.normal(0, 1, (1, 128)), rng.normal(0, 1, (1, 128))
    np.testing.assert_allclose(oracle.softmax_attention(rng.normal(0, 1, 128), k, v, 0.1), v[0], atol=1e-14)


def test_zero_query_is_mean_value():
    rng = np.random.default_rng(3)
    k, v = rng.normal(0, 1, (37, 128)), rng.normal(0, 1, (37, 128))
    np.testing.assert_allclose(oracle.softmax_attention(np.zeros(128), k, v, 1.0), v.mean(0), atol=1e-13)


def test_matches_scipy_softmax_and_large_logits():
    rng = np.random.default_rng(4)
    k, v = rng.normal(0, 30, (300, 128)), rng.normal(0, 1, (300, 128))
    q = rng.normal(0, 1, 128)
    s = 1.0 / math.sqrt(128)
    ref = special.softmax(s * (k @ q)) @ v
    np.testing.assert_allclose(oracle.softmax_attention(q, k, v, s), ref, rtol=1e-12, atol=1e-14)


def test_rotated_space_identity():
    """q . (n Pi^T y) = n (Pi q) . y : logits can be taken against rotated queries."""
    rng = np.random.default_rng(5)
    pi = oracle.rotation_for(0, 0, 0, 0, 2, 32)
    q, y = rng.normal(0, 1, 32), rng.normal(0, 1, 32)
    assert abs(q @ (2.5 * (pi.T @ y)) - 2.5 * ((pi @ q) @ y)) <= 1e-12


def test_decode_attention_head_mapping_and_empty():
    rng = np.random.default_rng(6)
    q16 = rng.normal(0, 1, (4, 128)).astype(np.float16)
    kh, vh = rng.normal(0, 1, (10, 2, 128)), rng.normal(0, 1, (10, 2, 128))
    o = oracle.decode_attention(q16, kh, vh, 10)
    q = q16.astype(np.float64)
    np.testing.assert_allclose(o[3], oracle.softmax_attention(q[3], kh[:, 1], vh[:, 1], 1 / math.sqrt(128)))
    np.testing.assert_allclose(o[1], oracle.softmax_attention(q[1], kh[:, 0], vh[:, 0], 1 / math.sqrt(128)))
    assert np.all(oracle.decode_attention(q16, kh, vh, 0) == 0.0)


def test_buffered_positions_mask():
    np.testing.assert_array_equal(oracle.buffered_positions(10, 2, 3),
                                  [1, 1, 0, 0, 0, 0, 0, 1, 1, 1])
    assert oracle.buffered_positions(5, 4, 128).all()          # window covers everything
    assert not oracle.buffered_positions(6, 0, 0).any()
    np.testing.assert_array_equal(oracle.buffered_positions(6, 0, 2), [0, 0, 0, 0, 1, 1])
    assert oracle.buffered_positions(0, 4, 128).size == 0


def test_buffered_attention_brute_force():
    """Tiny case by explicit loops: fp16 key/value for sink and window tokens, dequantised otherwise."""
    rng = np.random.default_rng(11)
    t_len, hkv, g, d = 10, 2, 2, 128
    k16 = rng.normal(0, 1, (t_len, hkv, d)).astype(np.float16)
    v16 = rng.normal(0, 1, (t_len, hkv, d)).astype(np.float16)
    kh = k16.astype(np.float64) + rng.normal(0, 0.3, k16.shape)
    vh = v16.astype(np.float64) + rng.normal(0, 0.3, v16.shape)
    q = rng.normal(0, 1, (hkv * g, d)).astype(np.float16)
    got = oracle.decode_attention_buffered(q, k16, v16, kh, vh, 9, 2, 3)
    for h in range(hkv * g):
        kv = h // g
        w, acc = [], np.zeros(d)
        for t in range(9):
            exact = t < 2 or t >= 6
            kt = [float(x) for x in k16[t, kv]] if exact else list(kh[t, kv])
            w.append(sum(float(a) * b for a, b in zip(q[h], kt)) / math.sqrt(d))
        mx = max(w)
        e = [math.exp(x - mx) for x in w]
        for t in range(9):
            vt = v16[t, kv].astype(np.float64) if (t < 2 or t >= 6) else vh[t, kv]
            acc += e[t] * vt
        np.testing.assert_allclose(got[h], acc / sum(e), rtol=1e-12, atol=1e-13)


def test_buffered_attention_special_cases():
    rng = np.random.default_rng(12)
    t_len, hkv, d = 40, 1, 128
    k16 = rng.normal(0, 1, (t_len, hkv, d)).astype(np.float16)
    v16 = rng.normal(0, 1, (t_len, hkv, d)).astype(np.float16)
    kh = rng.normal(0, 1, k16.shape)
    vh = rng.normal(0, 1, v16.shape)
    q = rng.normal(0, 1, (2, d)).astype(np.float16)
    # no buffer: the packed-cache result
    np.testing.assert_array_equal(oracle.decode_attention_buffered(q, k16, v16, kh, vh, 40, 0, 0),
                                  oracle.decode_attention(q, kh, vh, 40))
    # buffer covering the whole sequence: plain fp16 attention
    np.testing.assert_array_equal(oracle.decode_attention_buffered(q, k16, v16, kh, vh, 30, 4, 128),
                                  oracle.decode_attention(q, k16.astype(np.float64), v16.astype(np.float64), 30))
    # a lossless cache makes the buffer irrelevant
    np.testing.assert_allclose(
        oracle.decode_attention_buffered(q, k16, v16, k16.astype(np.float64), v16.astype(np.float64), 40, 4, 8),
        oracle.decode_attention(q, k16.astype(np.float64), v16.astype(np.float64), 40), rtol=0, atol=0)
    # empty sequence
    assert np.all(oracle.decode_attention_buffered(q, k16, v16, kh, vh, 0, 4, 128) == 0.0)
