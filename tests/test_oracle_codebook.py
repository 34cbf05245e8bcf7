"""Pins of the oracle's Lloyd-Max codebooks against mathematics and published tables."""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate, stats

import oracle


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_symmetry_and_middle_threshold(b):
    c, t, d, _ = oracle.lloyd_max(b)
    assert len(c) == 2 ** b and len(t) == 2 ** b - 1
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    np.testing.assert_array_equal(c, -c[::-1])
    mid = t[len(t) // 2]
    assert mid == 0.0 and math.copysign(1.0, mid) == 1.0


def test_one_bit_closed_form():
    c, t, d, _ = oracle.lloyd_max(1)
    assert abs(c[1] - math.sqrt(2.0 / math.pi)) <= 1e-14
    assert abs(d - (1.0 - 2.0 / math.pi)) <= 1e-14


@pytest.mark.parametrize("b", [2, 3, 4])
def test_centroid_and_nearest_neighbour_conditions_by_quadrature(b):
    """Each output is the conditional mean of its cell (scipy quadrature, not the oracle's formula)."""
    c, t, d, _ = oracle.lloyd_max(b)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    for k in range(len(c)):
        mass = stats.norm.cdf(edges[k + 1]) - stats.norm.cdf(edges[k])
        mean = integrate.quad(lambda x: x * stats.norm.pdf(x), edges[k], edges[k + 1],
                              epsabs=1e-14, epsrel=1e-13)[0] / mass
        assert abs(mean - c[k]) <= 1e-9
    np.testing.assert_allclose(t, 0.5 * (c[1:] + c[:-1]), rtol=0, atol=1e-15)


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_distortion_by_quadrature(b):
    c, t, d, _ = oracle.lloyd_max(b)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    mse = sum(integrate.quad(lambda x, ck=ck: (x - ck) ** 2 * stats.norm.pdf(x), edges[k], edges[k + 1],
                             epsabs=1e-14, epsrel=1e-13)[0] for k, ck in enumerate(c))
    assert abs(mse - d) <= 1e-10


def test_distortion_table_decreasing_convex():
    dist = oracle.distortion_table()
    assert dist[0] == 1.0
    dd = -np.diff(dist)
    assert np.all(dd > 0) and np.all(np.diff(dd) < 0)


def test_against_max_1960_table(golden_dir):
    with open(os.path.join(golden_dir, "max1960_gaussian.json")) as f:
        g = json.load(f)["levels"]
    for b in range(1, 5):
        c, t, d, _ = oracle.lloyd_max(b)
        ref = g[str(b)]
        np.testing.assert_allclose(t[len(t) // 2:], ref["thresholds"], atol=1e-3)
        np.testing.assert_allclose(c[len(c) // 2:], ref["outputs"], atol=1e-3)
        assert abs(d - ref["mse"]) / ref["mse"] < 2e-3
