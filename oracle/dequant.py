"""Reconstruction of a packed vector (oracle; test infrastructure only).

MSE part [softpro §1.2, stage 1] (ast-softpro.ru, "Технология TurboQuant и её
применение с локальными LLM", section 1.2): x_mse = Pi^T (nu16 * c[idx]).

Residual part [softpro §1.2, stage 2]: only sign(S r) and ||r||_2 are kept, and
the page says ||r||_2 is the scale used for reconstruction but prints no
formula.  Reading: r_hat = sqrt(pi/2) / m * rho16 * S^T (2 sgn - 1).  For a
Gaussian row s, E[s sign(s.r)] = sqrt(2/pi) r / ||r||, so this is the only
scaling for which E_S <q, r_hat> = <q, r> (the QJL correction is an unbiased
inner-product estimate).  With the sign sketch off only the MSE part is used.
"""
from __future__ import annotations

import numpy as np


def dequantize(idx, sgn, nu16, rho16, rot, proj, codebook):
    """x_hat[N, d] in float64 from codes, signs (or None), and stored scales."""
    c = np.asarray(codebook["centroids"], dtype=np.float64)
    rot = np.asarray(rot, dtype=np.float64)
    z_hat = np.asarray(nu16, dtype=np.float64)[:, None] * c[np.asarray(idx, dtype=np.int64)]
    x_hat = z_hat @ rot                                  # Pi^T z_hat, row form
    if sgn is not None:
        proj = np.asarray(proj, dtype=np.float64)
        m = proj.shape[0]
        pm = np.where(np.asarray(sgn, dtype=bool), 1.0, -1.0)
        kappa = np.sqrt(np.pi / 2.0) / m
        x_hat = x_hat + kappa * np.asarray(rho16, dtype=np.float64)[:, None] * (pm @ proj)
    return x_hat
