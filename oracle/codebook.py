"""Lloyd-Max scalar quantizer for a Gaussian (oracle; test infrastructure only).

[kiosk "Как работает"] = kiosknews.app, "3 бита вместо 16: разбираем TurboQuant
и когда его реально стоит включать", section "Как работает TurboQuant": the
grid is the Lloyd-Max quantizer of the known post-rotation distribution,
computed once and stored, with no calibration.
[softpro §1.2] = ast-softpro.ru, "Технология TurboQuant и её применение с
локальными LLM", section 1.2, stage 1: an MSE-optimal scalar quantizer with
b-1 bits per coordinate.

Reading: the distribution is N(0, sigma^2) with sigma = 1/sqrt(d), the law a
coordinate of a randomly rotated unit vector approaches; the page's mention of
beta distributions concerns the exact finite-d law, which is not used here.

Lloyd-Max alternates the two optimality conditions of an MSE quantizer:
thresholds are midpoints of neighbouring centroids, and each centroid is the
conditional mean of its cell.  For the Gaussian the conditional mean of
[a, b) is sigma * (phi(a/s) - phi(b/s)) / (Phi(b/s) - Phi(a/s)).
"""
from __future__ import annotations

import numpy as np
from scipy.special import ndtr, ndtri


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
