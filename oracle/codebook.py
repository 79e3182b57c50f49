"""Lloyd-Max scalar quantizer for a Gaussian (oracle; test infrastructure only).

[kiosk "Как работает"] = kiosknews.app, "3 бита вместо 16: разбираем TurboQuant
и когда его реально стоит включать", section "Как работает TurboQuant": the
grid is the Lloyd-Max quantizer of the known post-rotation distribution,
computed once and stored, with no calibration.
[softpro §1.2] = ast-softpro.ru, "Технология TurboQuant и её применение с
локальными LLM", section 1.2, stage 1: an MSE-optimal scalar quantizer with
b-1 bits per coordinate.

Reading: by default the distribution is N(0, sigma^2) with sigma = 1/sqrt(d),
the law a coordinate of a randomly rotated unit vector approaches.  The page's
theory is stated with beta distributions: the exact finite-d law of such a
coordinate, u^2 ~ Beta(1/2, (d-1)/2), is the alternative `build_codebook_sphere`.

Lloyd-Max alternates the two optimality conditions of an MSE quantizer:
thresholds are midpoints of neighbouring centroids, and each centroid is the
conditional mean of its cell.  For the Gaussian the conditional mean of
[a, b) is sigma * (phi(a/s) - phi(b/s)) / (Phi(b/s) - Phi(a/s)).
"""
from __future__ import annotations

import numpy as np
from scipy.special import betainc, betaln, ndtr, ndtri


def _phi(x):
    return np.exp(-0.5 * x * x) / np.sqrt(2.0 * np.pi)


def _cell_prob(a, b):
    """P(a <= X < b) for X ~ N(0,1), computed on the side of the smaller tail."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    upper = a > 0  # both ends in the right half: use survival functions
    return np.where(upper, ndtr(-a) - ndtr(-b), ndtr(b) - ndtr(a))


def build_codebook(bits_mse: int, sigma: float, tol: float = 1e-15, max_iter: int = 100000):
    """Return dict(centroids[L], boundaries[L-1], mse, iterations) in units of x.

    centroids ascending; boundaries[k-1] separates cell k-1 from cell k.
    mse is the expected squared error per coordinate, sigma^2 (1 - sum P_k c_k^2 / sigma^2).
    """
    if bits_mse < 1 or bits_mse > 3:
        raise ValueError("bits_mse must be 1, 2 or 3")
    L = 1 << bits_mse
    # start from the quantiles at the middle of L equal-probability cells
    c = ndtri((np.arange(L) + 0.5) / L)          # N(0,1) units
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate([[-np.inf], t])
        hi = np.concatenate([t, [np.inf]])
        num = _phi(lo) - _phi(hi)
        den = _cell_prob(lo, hi)
        c_new = num / den
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta <= tol:
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    # symmetric density: enforce exact antisymmetry of the centroids
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate([[-np.inf], t])
    hi = np.concatenate([t, [np.inf]])
    P = _cell_prob(lo, hi)
    mse = 1.0 - float(np.sum(P * c * c))
    return {
        "bits_mse": bits_mse,
        "levels": L,
        "sigma": float(sigma),
        "centroids": c * sigma,
        "boundaries": t * sigma,
        "mse": mse * sigma * sigma,
        "iterations": it,
    }


# ------------------------------------------- exact law of a unit-vector coordinate --
# u = one coordinate of a uniformly random unit vector in R^d (d >= 3):
# density f(u) = (1 - u^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1].
# P(u >= x) = I_{1-x^2}((d-1)/2, 1/2) / 2 for x >= 0 (u^2 ~ Beta(1/2, (d-1)/2)),
# and int_a^b u f(u) du = g(a) - g(b) with g(u) = (1 - u^2)^((d-1)/2) / ((d-1) B).

def _sphere_tail(x, d):
    x = np.asarray(x, dtype=np.float64)
    q = 0.5 * (d - 1)
    return np.where(x >= 1.0, 0.0, 0.5 * betainc(q, 0.5, np.clip(1.0 - x * x, 0.0, 1.0)))


def _sphere_prob(a, b, d):
    """P(a < u <= b), from the tail on the side of each end."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_pos = _sphere_tail(a, d) - _sphere_tail(b, d)
    both_neg = _sphere_tail(-b, d) - _sphere_tail(-a, d)
    straddle = 1.0 - _sphere_tail(-a, d) - _sphere_tail(b, d)
    return np.where(a >= 0, both_pos, np.where(b <= 0, both_neg, straddle))


def _sphere_g(u, d):
    u = np.asarray(u, dtype=np.float64)
    q = 0.5 * (d - 1)
    inside = np.abs(u) < 1.0
    val = np.exp(q * np.log1p(-np.where(inside, u * u, 0.0)) - np.log(2.0 * q) - betaln(0.5, q))
    return np.where(inside, val, 0.0)


def build_codebook_sphere(bits_mse: int, d: int, tol: float = 1e-13, max_iter: int = 100000):
    """Lloyd-Max for the exact law of one coordinate of a random unit vector in R^d.

    Same conditions and symmetrization as build_codebook; centroids and
    boundaries in absolute u units; mse = E[(u - c(u))^2] = 1/d - sum P_k c_k^2.
    tol is in units of sigma = 1/sqrt(d).
    """
    if bits_mse < 1 or bits_mse > 3:
        raise ValueError("bits_mse must be 1, 2 or 3")
    if d < 3:
        raise ValueError("d must be at least 3")
    L = 1 << bits_mse
    sigma = 1.0 / np.sqrt(d)
    c = np.clip(ndtri((np.arange(L) + 0.5) / L) * sigma, -0.999, 0.999)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate([[-1.0], t])
        hi = np.concatenate([t, [1.0]])
        c_new = (_sphere_g(lo, d) - _sphere_g(hi, d)) / _sphere_prob(lo, hi, d)
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta <= tol * sigma:
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    lo = np.concatenate([[-1.0], t])
    hi = np.concatenate([t, [1.0]])
    P = _sphere_prob(lo, hi, d)
    return {
        "bits_mse": bits_mse,
        "levels": L,
        "sigma": float(sigma),
        "centroids": c,
        "boundaries": t,
        "mse": 1.0 / d - float(np.sum(P * c * c)),
        "iterations": it,
    }
