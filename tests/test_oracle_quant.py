"""Pins of the oracle's encoder, decoder, fp16 norm rounding and bit layout."""
import math
import struct

import numpy as np
import pytest

import oracle
from oracle import layout, quant


def test_f16_single_rounding_matches_struct():
    """numpy's float64 -> float16 cast and Python's binary16 packing (both one RNE step) agree."""
    rng = np.random.default_rng(0)
    xs = list(np.exp(rng.normal(0, 4, 2000)) * rng.choice([-1, 1], 2000))
    # exact ties between fp16 neighbours, and values just off a tie (double rounding traps)
    for base in (1.0, 3.0, 1000.0, 6.1e-5):
        ulp = np.spacing(np.float16(base)).astype(np.float64)
        xs += [base + ulp / 2, base + 1.5 * ulp, base + ulp / 2 + 2.0 ** -40, base + ulp / 2 - 2.0 ** -40]
    xs = [x for x in xs if abs(x) < 65504]
    got = oracle.f16_bits(np.array(xs))
    ref = np.array([struct.unpack("<H", struct.pack("<e", x))[0] for x in xs], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_groups_order_and_pairing():
    bits = np.zeros(64, np.int8)
    bits[[3, 10]] = 4
    bits[[0]] = 1
    bits[[5, 6, 7]] = 2
    g = oracle.groups_for(bits)
    assert [w for w, _ in g] == [4, 2, 1]
    np.testing.assert_array_equal(g[0][1], [3, 67, 10, 74])
    np.testing.assert_array_equal(g[1][1], [5, 69, 6, 70, 7, 71])
    np.testing.assert_array_equal(g[2][1], [0, 64])


def test_groups_interleaved_pairing():
    bits = np.zeros(64, np.int8)
    bits[[3, 10]] = 4
    bits[[0]] = 1
    bits[[5, 6, 7]] = 2
    g = oracle.groups_for(bits, "interleaved")
    assert [w for w, _ in g] == [4, 2, 1]
    np.testing.assert_array_equal(g[0][1], [6, 7, 20, 21])
    np.testing.assert_array_equal(g[1][1], [10, 11, 12, 13, 14, 15])
    np.testing.assert_array_equal(g[2][1], [0, 1])
    with pytest.raises(ValueError):
        oracle.groups_for(bits, "other")


def test_interleaved_encode_equals_half_split_on_moved_coordinates():
    """A key with its (j, j+64) pairs moved to (2j, 2j+1) encodes to the same codes and norms
    under the interleaved pairing, and decodes to the moved reconstruction."""
    rng = np.random.default_rng(3)
    bits = np.zeros(64, np.int8)
    bits[rng.permutation(64)[:48]] = rng.integers(1, 5, 48)
    x = (rng.normal(0, 1, (50, 128)) * np.exp(rng.normal(0, 1, 128))).astype(np.float16)
    xi = np.empty_like(x)
    xi[:, 0::2], xi[:, 1::2] = x[:, :64], x[:, 64:]
    c_h, n_h = oracle.encode_k(x, bits, 7, 2, 1)
    c_i, n_i = oracle.encode_k(xi, bits, 7, 2, 1, pairing="interleaved")
    np.testing.assert_array_equal(c_i, c_h)
    np.testing.assert_array_equal(n_i, n_h)
    r_h = oracle.dequant_k(c_h, n_h, bits, 7, 2, 1)
    r_i = oracle.dequant_k(c_i, n_i, bits, 7, 2, 1, pairing="interleaved")
    np.testing.assert_array_equal(r_i[:, 0::2], r_h[:, :64])
    np.testing.assert_array_equal(r_i[:, 1::2], r_h[:, 64:])


def test_hand_worked_two_dim_group():
    """x = (3, 4), identity rotation, 2 bits: n = 5, z = sqrt(2) * (0.6, 0.8) -> codes (2, 3)."""
    x = np.array([[3.0, 4.0]], np.float16)
    codes, norms = quant.encode_groups(x, [(2, np.array([0, 1]))], [np.eye(2)])
    assert norms[0, 0] == 5.0
    np.testing.assert_array_equal(codes[0], [2, 3])
    c2 = oracle.lloyd_max(2)[0]
    np.testing.assert_allclose(5.0 * c2[[2, 3]] / math.sqrt(2), [1.60085, 5.34015], atol=1e-4)


def test_zero_vector_codes_and_norm():
    bits = np.full(64, 3, np.int8)
    codes, slots = oracle.encode_k(np.zeros((2, 128), np.float16), bits, 0, 0, 0)
    assert np.all(codes == 3) and np.all(slots == 0)
    vc, vn = oracle.encode_v(np.zeros((1, 128), np.float16), 2, 0, 0, 0)
    assert np.all(vc == 1) and np.all(vn == 0)
    xh = oracle.dequant_k(codes, slots, bits, 0, 0, 0)
    assert np.all(xh == 0.0)


@pytest.mark.parametrize("d", [2, 8, 32, 128])
def test_distortion_decreases_with_bits(d):
    rng = np.random.default_rng(d)
    x = rng.normal(0, 1, (4000, d)).astype(np.float16).astype(np.float64)
    errs = []
    for b in range(1, 5):
        pi = oracle.rotation_for(0, 0, 0, 0, b, d)
        coords = np.arange(d)
        codes, norms = quant.encode_groups(x.astype(np.float16), [(b, coords)], [pi])
        c = oracle.lloyd_max(b)[0]
        xh = norms[:, :1] * ((c[codes] / math.sqrt(d)) @ pi)
        errs.append(np.mean(np.sum((x - xh) ** 2, 1) / np.sum(x ** 2, 1)))
    assert all(errs[i] > errs[i + 1] for i in range(3)), errs


def test_distortion_at_128_matches_codebook():
    """At d_g = 128 the rotated coordinates are close to N(0, 1/d), so the MSE is near D(b)."""
    rng = np.random.default_rng(1)
    d, n = 128, 100000
    x16 = rng.normal(0, 1, (n, d)).astype(np.float16)
    x = x16.astype(np.float64)
    dist = oracle.distortion_table()
    for b in range(1, 5):
        codes, vn = oracle.encode_v(x16, b, 0, 0, 0)
        xh = oracle.dequant_v(codes, vn, b, 0, 0, 0)
        e = np.mean(np.sum((x - xh) ** 2, 1) / np.sum(x ** 2, 1))
        assert abs(e - dist[b]) / dist[b] < 0.05, (b, e, dist[b])


def test_pack_roundtrip_random_widths():
    rng = np.random.default_rng(2)
    widths = rng.integers(1, 5, 150)
    widths[:20] = 3                       # many straddling 3-bit codes
    n_words = (int(widths.sum()) + 31) // 32
    codes = (rng.integers(0, 16, (40, 150)) & ((1 << widths) - 1)).astype(np.uint8)
    words = layout.pack_bits(codes, widths, n_words)
    np.testing.assert_array_equal(layout.unpack_bits(words, widths), codes)


def test_pack_hand_example():
    """Codes 0xA (4b), 0x5 (3b), 0x7 (3b), ... LSB-first; the 11th 3-bit code straddles words."""
    widths = np.array([4] + [3] * 10 + [2])
    codes = np.array([[0xA, 5, 7, 1, 0, 2, 3, 4, 6, 5, 7, 2]], np.uint8)
    w = layout.pack_bits(codes, widths, 2)
    bits = "".join(format(int(c), "0%db" % int(wd))[::-1] for c, wd in zip(codes[0], widths))
    val = int(bits[::-1], 2)
    assert int(w[0, 0]) == val & 0xFFFFFFFF and int(w[0, 1]) == val >> 32
    assert int(w[0, 0]) & 0xF == 0xA and (int(w[0, 0]) >> 4) & 7 == 5
    # code 10 (value 7) sits at bits 31..33
    assert (int(w[0, 0]) >> 31) & 1 == 1 and int(w[0, 1]) & 3 == 3


def test_k_and_v_layout_roundtrip_ragged():
    rng = np.random.default_rng(4)
    bits = oracle.greedy_allocate(np.exp(rng.normal(0, 2, 64)), 3, oracle.distortion_table())
    t = 150
    k16 = rng.normal(0, 1, (t, 128)).astype(np.float16)
    codes, slots = oracle.encode_k(k16, bits, 0, 0, 0)
    assert oracle.k_words_per_token(bits) == 12
    karr, knrm = layout.pack_k(codes, slots, bits, 3)
    assert karr.shape == (3, 12, 64) and knrm.shape == (3, 64, 4)
    assert np.all(karr[2, :, t - 128:] == 0)
    c2, s2 = layout.unpack_k(karr, knrm, bits, t)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, slots)
    for vb in (1, 2, 3, 4):
        vc, vn = oracle.encode_v(k16, vb, 0, 0, 0)
        varr, vnrm = layout.pack_v(vc, vn, vb, 3)
        assert varr.shape == (3, 128, 2 * vb)
        c3, n3 = layout.unpack_v(varr, vnrm, vb, t)
        np.testing.assert_array_equal(c3, vc)
        np.testing.assert_array_equal(n3, vn)


def test_v_layout_token_lane_bits():
    """Coordinate i of tile 0: token lane l's code sits at bits [b*l, b*(l+1))."""
    codes = np.zeros((64, 128), np.uint8)
    codes[10, 5] = 3
    codes[63, 127] = 2
    varr, _ = layout.pack_v(codes, np.zeros(64, np.uint16), 2, 1)
    assert varr[0, 5, 0] == 3 << 20
    assert varr[0, 127, 3] == 2 << 30


@pytest.mark.parametrize("widths", [(4, 2), (3, 1)])
def test_dequant_k_roundtrip_per_group_distortion(widths):
    """dequant_k(encode_k(x)) over a two-group allocation (d_g = 64 each): every group's relative
    error is within 5% of the codebook's D(b).  Each group's coordinates carry their own scale
    (x 1 and x 1000), so a wrong norm slot, a wrong scatter of the group coordinates or an
    un-rotation by Pi instead of Pi^T moves the error far outside the bound."""
    rng = np.random.default_rng(6 + widths[0])
    bits = np.zeros(64, np.int8)
    perm = rng.permutation(64)
    bits[perm[:32]], bits[perm[32:]] = widths
    n = 40000
    x = rng.normal(0, 1, (n, 128))
    groups = oracle.groups_for(bits)
    x[:, groups[1][1]] *= 1000.0
    x16 = x.astype(np.float16)
    codes, slots = oracle.encode_k(x16, bits, 3, 1, 2)
    xh = oracle.dequant_k(codes, slots, bits, 3, 1, 2)
    xf = x16.astype(np.float64)
    dist = oracle.distortion_table()
    for w, coords in groups:
        e = np.mean(np.sum((xf[:, coords] - xh[:, coords]) ** 2, 1) / np.sum(xf[:, coords] ** 2, 1))
        assert abs(e - dist[w]) / dist[w] < 0.05, (w, e, dist[w])
    zero = np.setdiff1d(np.arange(128), np.concatenate([c for _, c in groups]))
    assert zero.size == 0 or np.all(xh[:, zero] == 0.0)


def test_dequant_k_four_groups_at_32():
    """Four groups of 16 blocks (d_g = 32): each group's error is within 8% of D(b) (the N(0, 1/d)
    codebook sits a few per cent off the exact marginal at d = 32), and the norms of the four
    slots, scaled apart by powers of ten, each reconstruct their own group."""
    rng = np.random.default_rng(5)
    bits = np.zeros(64, np.int8)
    perm = rng.permutation(64)
    for i, w in enumerate((4, 3, 2, 1)):
        bits[perm[16 * i:16 * (i + 1)]] = w
    x = rng.normal(0, 1, (20000, 128))
    groups = oracle.groups_for(bits)
    for w, coords in groups:
        x[:, coords] *= 10.0 ** (w - 1)
    x16 = x.astype(np.float16)
    codes, slots = oracle.encode_k(x16, bits, 0, 4, 1)
    xh = oracle.dequant_k(codes, slots, bits, 0, 4, 1)
    xf = x16.astype(np.float64)
    dist = oracle.distortion_table()
    for w, coords in groups:
        e = np.mean(np.sum((xf[:, coords] - xh[:, coords]) ** 2, 1) / np.sum(xf[:, coords] ** 2, 1))
        assert abs(e - dist[w]) / dist[w] < 0.08, (w, e, dist[w])


def test_dequant_k_hand_worked_two_groups():
    """Block 0 at 4 bits (coordinates 0, 64), blocks 1 and 2 at 2 bits (1, 65, 2, 66), the rest 0.
    Rotations given explicitly: a 2 x 2 rotation Pi = [[0.6, -0.8], [0.8, 0.6]] for the 4-bit
    group (x_hat = n Pi^T y_hat, not n Pi y_hat) and the identity for the 2-bit group.  Norm slots
    4 - w: slot 0 = 2, slot 2 = 0.5; slots 1 and 3 hold 7 and 9 and must not be read."""
    bits = np.zeros(64, np.int8)
    bits[0] = 4
    bits[[1, 2]] = 2
    pi4 = np.array([[0.6, -0.8], [0.8, 0.6]])
    rots = [pi4, np.eye(4)]
    codes = np.array([[3, 12, 0, 3, 1, 2]], np.uint8)
    slots = oracle.f16_bits(np.array([[2.0, 7.0, 0.5, 9.0]]))
    got = oracle.dequant_k(codes, slots, bits, 0, 0, 0, rots=rots)
    c4, c2 = oracle.lloyd_max(4)[0], oracle.lloyd_max(2)[0]
    a, b = c4[3] / math.sqrt(2), c4[12] / math.sqrt(2)
    want = np.zeros(128)
    want[0], want[64] = 2.0 * (0.6 * a + 0.8 * b), 2.0 * (-0.8 * a + 0.6 * b)
    want[[1, 65, 2, 66]] = 0.5 * c2[[0, 3, 1, 2]] / 2.0
    np.testing.assert_allclose(got[0], want, rtol=0, atol=1e-15)
    # the centroids used, against the printed 4-bit Lloyd-Max values (+-1.2562 for codes 3 and 12,
    # +-0.4528 and +-1.5104 for the 2-bit codes)
    assert abs(c4[3] + 1.2562) < 5e-4 and abs(c4[12] - 1.2562) < 5e-4
    assert abs(c2[0] + 1.5104) < 5e-4 and abs(c2[1] + 0.4528) < 5e-4


def test_k_layout_word_major_hand_placed():
    """Key array [tile][word][lane]: token t's stream word k sits at [t // 64, k, t % 64]; its
    norm slots at [t // 64, t % 64, slot].  Token 70 (tile 1, lane 6) with the 4-bit code 0xB at
    stream position 0 (bits 0..3 of word 0) and the 2-bit code 2 at position 8, the first code after
    the 32 bits of the 4-bit group (bits 0..1 of word 1); everything else 0."""
    bits = np.full(64, 2, np.int8)
    bits[:4] = 4
    bits[4:8] = 0                           # 8 coordinates of 4 bits, 112 of 2 bits: 256 bits
    assert oracle.k_words_per_token(bits) == 8
    codes = np.zeros((100, 120), np.uint8)
    codes[70, 0], codes[70, 8] = 0xB, 0x2
    slots = np.zeros((100, 4), np.uint16)
    slots[70] = [0x3C00, 0, 0x4000, 0]
    karr, knrm = layout.pack_k(codes, slots, bits, 2)
    assert karr[1, 0, 6] == 0xB and karr[1, 1, 6] == 0x2
    karr[1, 0, 6] = karr[1, 1, 6] = 0
    assert not karr.any()
    np.testing.assert_array_equal(knrm[1, 6], [0x3C00, 0, 0x4000, 0])
    knrm[1, 6] = 0
    assert not knrm.any()
