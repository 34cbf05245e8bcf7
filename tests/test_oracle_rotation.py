"""Pins of the oracle's seeded stream and Haar rotations."""
import json
import math
import os

import numpy as np
from scipy import stats

import oracle
from oracle.rotation import gaussian_matrix


def test_splitmix64_reference_vector(golden_dir):
    with open(os.path.join(golden_dir, "splitmix64.json")) as f:
        g = json.load(f)
    gen = oracle.SplitMix64(g["state"])
    assert [gen.next() for _ in range(5)] == [int(v) for v in g["outputs"]]


def test_absorb_is_one_step_from_xored_state():
    a = oracle.SplitMix64(0)
    a.absorb(1234567 ^ 0)
    b = oracle.SplitMix64(1234567)
    assert a.state == b.next()


def test_uniform_range_and_resolution():
    gen = oracle.SplitMix64(7)
    us = [gen.uniform() for _ in range(20000)]
    assert min(us) >= 0.0 and max(us) < 1.0
    assert all((u * 2 ** 53).is_integer() for u in us[:1000])
    assert stats.kstest(us, "uniform").pvalue > 1e-4


def test_box_muller_radius_identity_and_normality():
    gen = oracle.seeded_stream(1, 2, 3, 0, 3, 8)
    ref = oracle.seeded_stream(1, 2, 3, 0, 3, 8)
    z = gaussian_matrix(gen, 128).reshape(-1)
    for i in range(0, 200, 2):
        u1 = ref.uniform()
        ref.uniform()
        assert abs(z[i] ** 2 + z[i + 1] ** 2 - (-2.0 * math.log(1.0 - u1))) <= 1e-12 * (1 + z[i] ** 2 + z[i + 1] ** 2)
    assert stats.kstest(z, "norm").pvalue > 1e-4
    assert abs(z.mean()) < 0.03 and abs(z.var() - 1) < 0.03


def test_haar_is_q_of_qr_with_positive_diagonal():
    gen = oracle.seeded_stream(0, 0, 0, 0, 2, 24)
    g = gaussian_matrix(gen, 24)
    pi = oracle.haar_rotation(g)
    np.testing.assert_allclose(pi.T @ pi, np.eye(24), atol=1e-13)
    r = pi.T @ g                          # must be upper triangular with a positive diagonal
    assert np.abs(np.tril(r, -1)).max() <= 1e-12 * np.abs(g).max()
    assert np.all(np.diag(r) > 0)


def test_rotation_determinism_and_field_sensitivity():
    base = oracle.rotation_for(0, 0, 1, 0, 3, 16)
    np.testing.assert_array_equal(base, oracle.rotation_for(0, 0, 1, 0, 3, 16))
    for args in [(1, 0, 1, 0, 3, 16), (0, 1, 1, 0, 3, 16), (0, 0, 2, 0, 3, 16),
                 (0, 0, 1, 1, 3, 16), (0, 0, 1, 0, 2, 16)]:
        assert np.abs(oracle.rotation_for(*args) - base).max() > 0.1


def test_haar_first_moment():
    """E[Pi_00^2] = 1/d for Haar-distributed Pi."""
    d, n = 4, 1500
    vals = [oracle.rotation_for(s, 0, 0, 0, 1, d)[0, 0] ** 2 for s in range(n)]
    assert abs(np.mean(vals) - 1.0 / d) < 4 * np.std(vals) / math.sqrt(n)


def test_box_muller_order_from_reference_outputs(golden_dir):
    """The Gaussian fill, computed by hand from the published SplitMix64 outputs: pair k takes
    u1 = out[2k] >> 11 * 2^-53 and u2 = out[2k+1] >> 11 * 2^-53, z0 = r cos(2 pi u2) goes to
    element 2k and z1 = r sin(2 pi u2) to element 2k + 1 of the row-major matrix, with
    r = sqrt(-2 ln(1 - u1)).  A swapped cos / sin, swapped u1 / u2 or a column-major fill fails."""
    with open(os.path.join(golden_dir, "splitmix64.json")) as f:
        g = json.load(f)
    outs = [int(v) for v in g["outputs"]]
    u = [(o >> 11) * 2.0 ** -53 for o in outs[:4]]
    want = []
    for k in range(2):
        r = math.sqrt(-2.0 * math.log(1.0 - u[2 * k]))
        want += [r * math.cos(2.0 * math.pi * u[2 * k + 1]), r * math.sin(2.0 * math.pi * u[2 * k + 1])]
    z = gaussian_matrix(oracle.SplitMix64(g["state"]), 2)
    np.testing.assert_allclose(z, np.array(want).reshape(2, 2), rtol=0, atol=1e-15)
    assert z[0, 1] == want[1] and z[1, 0] == want[2]
