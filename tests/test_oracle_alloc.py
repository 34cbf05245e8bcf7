"""Pins of the oracle's energy and greedy allocation."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth


def _brute(e, budget, dist):
    best, best_sets = None, []
    for bits in itertools.product(range(5), repeat=len(e)):
        if sum(bits) != budget:
            continue
        obj = sum(ej * dist[b] for ej, b in zip(e, bits))
        if best is None or obj < best - 1e-15 * abs(best):
            best, best_sets = obj, [bits]
        elif abs(obj - best) <= 1e-15 * abs(best):
            best_sets.append(bits)
    return best, best_sets


@pytest.mark.parametrize("nb", [1, 2, 3, 4, 5])
def test_greedy_matches_brute_force(nb):
    dist = oracle.distortion_table()
    rng = np.random.default_rng(nb)
    for trial in range(6):
        e = np.exp(rng.normal(0, 2, nb))
        for budget_avg in range(0, 5):
            bits = oracle.greedy_allocate(e, budget_avg, dist)
            assert bits.sum() == budget_avg * nb and bits.min() >= 0 and bits.max() <= 4
            best, sets = _brute(e, budget_avg * nb, dist)
            obj = sum(ej * dist[b] for ej, b in zip(e, bits))
            assert abs(obj - best) <= 1e-12 * abs(best)
            if len(sets) == 1:
                assert tuple(bits) == sets[0]


def test_greedy_equals_top_b_marginal_gains():
    dist = oracle.distortion_table()
    dd = -np.diff(dist)
    rng = np.random.default_rng(11)
    e = np.exp(rng.normal(0, 1.5, 64))
    for avg in (1, 2, 3):
        gains = [(e[j] * dd[b], j, b) for j in range(64) for b in range(4)]
        top = sorted(gains, key=lambda g: -g[0])[:avg * 64]
        ref = np.zeros(64, np.int8)
        for _, j, _ in top:
            ref[j] += 1
        np.testing.assert_array_equal(oracle.greedy_allocate(e, avg, dist), ref)


def test_uniform_energy_gives_uniform_widths():
    dist = oracle.distortion_table()
    for avg in range(5):
        np.testing.assert_array_equal(oracle.greedy_allocate(np.ones(64), avg, dist), np.full(64, avg))


def test_greedy_tie_goes_to_lowest_block():
    dist = oracle.distortion_table()
    # third bit: blocks 0 and 1 tie at gain D(1) - D(2); block 0 wins
    bits = oracle.greedy_allocate(np.array([1.0, 1.0, 0.0]), 1, dist)
    np.testing.assert_array_equal(bits, [2, 1, 0])
    bits = oracle.greedy_allocate(np.array([2.0, 2.0, 0.0, 0.0]), 1, dist)
    # gains 2*0.636 twice, then 2*0.246 twice: all four bits go to blocks 0 and 1
    np.testing.assert_array_equal(bits, [2, 2, 0, 0])


def _random_f16(rng, shape):
    x = rng.normal(0, 1, shape) * np.exp(rng.normal(0, 3, shape))
    x = np.clip(x, -60000, 60000).astype(np.float16)
    x.flat[:5] = np.array([6.0e-8, -6.0e-8, 65504.0, 0.0, 1.0e-5], dtype=np.float16)
    return x


def test_exact_sum_squares_matches_fractions():
    rng = np.random.default_rng(3)
    x = _random_f16(rng, (20, 37))
    got = oracle.exact_sum_squares_f16(x, axis=1)
    for r in range(20):
        exact = sum(Fraction(float(v)) ** 2 for v in x[r])
        assert got[r] == float(exact)
        assert got[r] == math.fsum(float(v) ** 2 for v in x[r])


def test_energy_formula_on_constructed_inputs():
    """Two KV heads, G = 2; only known blocks carry mass, with exact expected values."""
    n, hkv, g = 4, 2, 2
    q = np.zeros((n, hkv * g, 128), np.float16)
    k = np.zeros((n, hkv, 128), np.float16)
    q[:, 0, 5] = 1.0          # head 0 group, block 5 (coordinate 5)
    q[:, 1, 69] = 2.0         # head 0 group, block 5 (coordinate 69)
    q[:, 3, 7] = 3.0          # head 1 group, block 7
    k[:, 0, 5] = 0.5
    k[:, 1, 71] = 4.0         # head 1, block 7 via coordinate 71
    e = oracle.energy(q, k, hkv)
    assert e.shape == (2, 64)
    # head 0 block 5: Eq = (4*1 + 4*4) / (4*2) = 2.5 ; Ek = 4*0.25/4 = 0.25
    assert e[0, 5] == 2.5 * 0.25
    # head 1 block 7: Eq = 4*9/8 = 4.5 ; Ek = 4*16/4 = 16
    assert e[1, 7] == 4.5 * 16.0
    e[0, 5] = 0.0
    e[1, 7] = 0.0
    assert np.all(e == 0.0)


def test_energy_matches_fraction_arithmetic():
    cfg = synth.small(2, n_cal=16)
    q, k = synth.calibration(cfg)
    e = oracle.energy(q, k, cfg.n_kv_heads)
    g = cfg.group
    for h, j in [(0, 0), (1, 17), (0, 63)]:
        sq = sum(Fraction(float(q[t, hh, c])) ** 2 for t in range(16)
                 for hh in range(h * g, (h + 1) * g) for c in (j, j + 64))
        sk = sum(Fraction(float(k[t, h, c])) ** 2 for t in range(16) for c in (j, j + 64))
        eq = float(sq) / float(16 * g)
        ek = float(sk) / 16.0
        assert e[h, j] == eq * ek


def test_energy_is_rope_invariant():
    """Block norms are RoPE-invariant: energies of pre- and post-RoPE inputs agree up to fp16 rounding."""
    rng = np.random.default_rng(5)
    q = rng.normal(0, 1, (256, 2, 128)) * np.exp(rng.normal(0, 1, 128))
    k = rng.normal(0, 1, (256, 1, 128)) * np.exp(rng.normal(0, 1, 128))
    pos = np.arange(256) * 37
    e_pre = oracle.energy(q.astype(np.float16), k.astype(np.float16), 1)
    e_post = oracle.energy(synth.rope_f64(q, pos, 1e4).astype(np.float16),
                           synth.rope_f64(k, pos, 1e4).astype(np.float16), 1)
    np.testing.assert_allclose(e_post, e_pre, rtol=2e-3)


def test_energy_interleaved_pairing_on_constructed_inputs():
    """Interleaved pairing: block j is coordinates (2j, 2j+1); mass at 10 and 11 lands in block 5."""
    n = 2
    q = np.zeros((n, 1, 128), np.float16)
    k = np.zeros((n, 1, 128), np.float16)
    q[:, 0, 10] = 1.0
    q[:, 0, 11] = 2.0
    k[:, 0, 11] = 3.0
    k[:, 0, 69] = 7.0          # block 34 (coordinates 68, 69); no query mass there
    e = oracle.energy(q, k, 1, pairing="interleaved")
    assert e[0, 5] == (2 * 1 + 2 * 4) / 2 * (2 * 9) / 2
    e[0, 5] = 0.0
    assert np.all(e == 0.0)
    # the same inputs read half-split put coordinate 10 in block 10 and 69 in block 5
    eh = oracle.energy(q, k, 1)
    assert eh[0, 10] == 0.0 and eh[0, 5] == 0.0 and eh[0, 11] == 4.0 * 9.0


def test_energy_interleaved_matches_fraction_arithmetic():
    cfg = synth.small(2, n_cal=16, pairing="interleaved")
    q, k = synth.calibration(cfg)
    e = oracle.energy(q, k, cfg.n_kv_heads, pairing="interleaved")
    g = cfg.group
    for h, j in [(0, 0), (1, 17), (0, 63)]:
        sq = sum(Fraction(float(q[t, hh, c])) ** 2 for t in range(16)
                 for hh in range(h * g, (h + 1) * g) for c in (2 * j, 2 * j + 1))
        sk = sum(Fraction(float(k[t, h, c])) ** 2 for t in range(16) for c in (2 * j, 2 * j + 1))
        assert e[h, j] == (float(sq) / float(16 * g)) * (float(sk) / 16.0)


def test_interleaved_config_is_a_coordinate_move_of_its_half_split_twin():
    """Both pairings see the same blocks: energies of the twin configs are identical."""
    half = synth.small(2, n_cal=64)
    inter = synth.small(2, n_cal=64, pairing="interleaved")
    qh, kh = synth.calibration(half)
    qi, ki = synth.calibration(inter)
    np.testing.assert_array_equal(qi[..., 0::2], qh[..., :64])
    np.testing.assert_array_equal(qi[..., 1::2], qh[..., 64:])
    np.testing.assert_array_equal(ki[..., 0::2], kh[..., :64])
    np.testing.assert_array_equal(oracle.energy(qi, ki, 2, pairing="interleaved"), oracle.energy(qh, kh, 2))
