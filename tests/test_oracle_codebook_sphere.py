"""Pins for the oracle's codebook of the exact unit-vector coordinate law.

u = one coordinate of a uniformly random unit vector in R^d has density
(1 - u^2)^((d-3)/2) / B(1/2, (d-1)/2); the method's theory is stated with beta
distributions (kiosknews.app, "3 бита вместо 16", section "Как работает
TurboQuant"), and u^2 ~ Beta(1/2, (d-1)/2).  Each pin is independent of the
oracle's own iteration: closed forms, quadrature, sampling, limits.
"""
import math

import numpy as np
import pytest
from scipy import integrate
from scipy.special import gammaln

from oracle import build_codebook, build_codebook_sphere


def _density(d):
    lnB = gammaln(0.5) + gammaln(0.5 * (d - 1)) - gammaln(0.5 * d)
    return lambda u: math.exp(0.5 * (d - 3) * math.log1p(-u * u) - lnB) if abs(u) < 1 else 0.0


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_d3_is_the_uniform_quantizer(bits):
    # d = 3: the coordinate is uniform on [-1, 1] (Archimedes), so Lloyd-Max is the
    # uniform quantizer: centroids (2k+1)/L - 1, boundaries 2k/L - 1, mse 1/(3 L^2)
    L = 1 << bits
    cb = build_codebook_sphere(bits, 3)
    k = np.arange(L)
    np.testing.assert_allclose(cb["centroids"], (2 * k + 1) / L - 1, atol=1e-12)
    np.testing.assert_allclose(cb["boundaries"], 2 * k[1:] / L - 1, atol=1e-12)
    assert abs(cb["mse"] - 1 / (3 * L * L)) < 1e-12


@pytest.mark.parametrize("d", [3, 4, 8, 64, 128, 256])
def test_one_bit_closed_form(d):
    # 1 bit: the centroid is E|u| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    cb = build_codebook_sphere(1, d)
    e_abs = math.exp(gammaln(0.5 * d) - gammaln(0.5 * (d + 1))) / math.sqrt(math.pi)
    np.testing.assert_allclose(cb["centroids"], [-e_abs, e_abs], rtol=1e-12)
    assert abs(cb["mse"] - (1 / d - e_abs * e_abs)) < 1e-14


@pytest.mark.parametrize("d", [5, 16, 128])
def test_density_normalization_and_variance(d):
    f = _density(d)
    mass = integrate.quad(f, -1, 1, epsabs=1e-14, limit=400)[0]
    var = integrate.quad(lambda u: u * u * f(u), -1, 1, epsabs=1e-14, limit=400)[0]
    assert abs(mass - 1) < 1e-10
    assert abs(var - 1 / d) < 1e-10


@pytest.mark.parametrize("bits", [1, 2, 3])
@pytest.mark.parametrize("d", [8, 128])
def test_centroid_and_midpoint_conditions_by_quadrature(bits, d):
    f = _density(d)
    cb = build_codebook_sphere(bits, d)
    c, t = cb["centroids"], cb["boundaries"]
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15)
    np.testing.assert_allclose(c, -c[::-1], atol=0)
    edges = [-1.0] + list(t) + [1.0]
    sigma = 1 / math.sqrt(d)
    for k in range(cb["levels"]):
        num = integrate.quad(lambda u: u * f(u), edges[k], edges[k + 1], epsabs=1e-16, epsrel=1e-13, limit=400)[0]
        den = integrate.quad(f, edges[k], edges[k + 1], epsabs=1e-16, epsrel=1e-13, limit=400)[0]
        assert abs(c[k] - num / den) <= 1e-10 * sigma, (k, c[k], num / den)


def test_distortion_by_sampling_unit_vectors():
    # draw random unit vectors in R^16 and quantize every coordinate
    d, bits = 16, 2
    cb = build_codebook_sphere(bits, d)
    rng = np.random.default_rng(1234)
    g = rng.standard_normal((200000, d))
    u = (g / np.linalg.norm(g, axis=1, keepdims=True)).ravel()
    idx = np.searchsorted(cb["boundaries"], u, side="right")
    err = (u - cb["centroids"][idx]) ** 2
    se = err.std() / math.sqrt(err.size)
    assert abs(err.mean() - cb["mse"]) < 4 * se, (err.mean(), cb["mse"], se)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_large_d_limit_is_the_gaussian_codebook(bits):
    d = 8192
    sigma = 1 / math.sqrt(d)
    s = build_codebook_sphere(bits, d)
    g = build_codebook(bits, sigma)
    # the coordinate law tends to N(0, 1/d) with O(1/d) corrections
    np.testing.assert_allclose(s["centroids"] / sigma, g["centroids"] / sigma, atol=5e-4)
    assert abs(s["mse"] / g["mse"] - 1) < 1e-3


@pytest.mark.parametrize("bits", [2, 3])
def test_optimal_for_its_own_law(bits):
    # under the exact law, the exact-law codebook has lower distortion than the
    # Gaussian codebook of the same sigma (both evaluated by quadrature)
    d = 8
    f = _density(d)

    def distortion(cb):
        edges = [-1.0] + list(cb["boundaries"]) + [1.0]
        return sum(integrate.quad(lambda u: (u - cb["centroids"][k]) ** 2 * f(u), edges[k], edges[k + 1],
                                  epsabs=1e-15, limit=400)[0] for k in range(cb["levels"]))

    s = build_codebook_sphere(bits, d)
    g = build_codebook(bits, 1 / math.sqrt(d))
    g["boundaries"] = np.clip(g["boundaries"], -1, 1)
    ds, dg = distortion(s), distortion(g)
    assert abs(ds - s["mse"]) < 1e-12
    assert ds < dg
