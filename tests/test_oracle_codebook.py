"""Pins for the oracle's Lloyd-Max codebook (independent of its own iteration)."""
import json
import math
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

from oracle import build_codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "max1960_gaussian.json")


def _cond_mean_quad(a, b, sigma):
    """E[X | a <= X < b], X ~ N(0, sigma^2), by numerical quadrature."""
    f = lambda x: norm.pdf(x, scale=sigma)
    num = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-16, epsrel=1e-14, limit=200)[0]
    den = integrate.quad(f, a, b, epsabs=1e-16, epsrel=1e-14, limit=200)[0]
    return num / den


@pytest.mark.parametrize("bits", [1, 2, 3])
@pytest.mark.parametrize("d", [128, 256])
def test_centroid_condition_by_quadrature(bits, d):
    sigma = 1 / math.sqrt(d)
    cb = build_codebook(bits, sigma)
    c, t = cb["centroids"], cb["boundaries"]
    edges = [-np.inf] + list(t) + [np.inf]
    for k in range(cb["levels"]):
        ref = _cond_mean_quad(edges[k], edges[k + 1], sigma)
        assert abs(c[k] - ref) <= 1e-12 * sigma + 1e-13 * abs(ref), (k, c[k], ref)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_midpoint_and_symmetry(bits):
    sigma = 1 / math.sqrt(128)
    cb = build_codebook(bits, sigma)
    c, t = cb["centroids"], cb["boundaries"]
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])
    for k in range(1, cb["levels"]):
        assert abs(t[k - 1] - 0.5 * (c[k - 1] + c[k])) <= 1e-15 * sigma
    assert t[cb["levels"] // 2 - 1] == 0.0


def test_one_bit_closed_form():
    # 1-bit Lloyd-Max for N(0, s^2): +-s*sqrt(2/pi), threshold 0, mse s^2 (1 - 2/pi)
    for d in (4, 128, 256):
        s = 1 / math.sqrt(d)
        cb = build_codebook(1, s)
        np.testing.assert_allclose(cb["centroids"], [-s * math.sqrt(2 / math.pi), s * math.sqrt(2 / math.pi)],
                                   rtol=1e-14)
        assert cb["boundaries"][0] == 0.0
        assert abs(cb["mse"] - s * s * (1 - 2 / math.pi)) < 1e-15


def _printed_tol(s):
    dec = len(s.split(".")[1]) if "." in s else 0
    return 1.5 * 10.0 ** (-dec) + 1e-9


@pytest.mark.parametrize("levels", ["2", "4", "8"])
def test_max_1960_table(levels):
    tab = json.load(open(GOLDEN))["levels"][levels]
    cb = build_codebook(int(math.log2(int(levels))), 1.0)
    L = cb["levels"]
    pos_c = cb["centroids"][L // 2:]
    pos_t = cb["boundaries"][L // 2 - 1:]
    for v, s in zip(pos_c, tab["outputs"]):
        assert abs(v - float(s)) <= _printed_tol(s), (v, s)
    for v, s in zip(pos_t, tab["thresholds"]):
        assert abs(v - float(s)) <= _printed_tol(s), (v, s)
    assert abs(cb["mse"] - float(tab["mse"])) <= _printed_tol(tab["mse"])


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_mse_by_quadrature_and_local_optimality(bits):
    sigma = 1 / math.sqrt(128)
    cb = build_codebook(bits, sigma)
    c = cb["centroids"]

    def mse_of(cent):
        t = 0.5 * (cent[:-1] + cent[1:])
        edges = [-np.inf] + list(t) + [np.inf]
        tot = 0.0
        for k in range(len(cent)):
            tot += integrate.quad(lambda x: (x - cent[k]) ** 2 * norm.pdf(x, scale=sigma),
                                  edges[k], edges[k + 1], epsabs=1e-18, limit=200)[0]
        return tot

    base = mse_of(c)
    assert abs(base - cb["mse"]) <= 1e-12 * sigma * sigma + 1e-10 * base
    # nudging any centroid (and re-deriving midpoints) cannot lower the distortion
    for k in range(len(c)):
        for eps in (1e-3, -1e-3):
            cc = c.copy()
            cc[k] += eps * sigma
            cc.sort()
            assert mse_of(cc) > base


def test_sigma_scaling():
    a = build_codebook(3, 1.0)
    b = build_codebook(3, 0.0625)
    np.testing.assert_allclose(b["centroids"], 0.0625 * a["centroids"], rtol=1e-13)
    np.testing.assert_allclose(b["boundaries"], 0.0625 * a["boundaries"], rtol=1e-13, atol=1e-18)
