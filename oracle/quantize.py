"""Per-vector quantizer (oracle; test infrastructure only).

Steps follow [softpro §1.2] = ast-softpro.ru, "Технология TurboQuant и её
применение с локальными LLM", section 1.2 "Как работает TurboQuant":

stage 1 ("Этап 1"): multiply each KV vector by a random orthogonal matrix, then
quantize each rotated coordinate independently with an MSE-optimal Lloyd-Max
quantizer of b-1 bits;
stage 2 ("Этап 2", QJL): form the residual r = x - DEQUANT_mse(Q_mse(x)),
project it with a random Gaussian matrix S, keep only sign(S r), and keep
||r||_2 as the reconstruction scale.

Readings (the pages leave these open):
* the quantizer acts on u = Pi x / ||x||; ||x|| is the per-vector norm, stored
  as fp16; the cell decision uses the unrounded norm, the reconstruction uses
  the stored one ([kiosk "Python + HuggingFace"]: kiosknews.app, "3 бита вместо
  16…", section "Python + HuggingFace" — quantize returns indices and norms);
* cell index = number of thresholds t_k with u >= t_k (a midpoint tie goes to
  the upper cell);
* DEQUANT_mse(Q_mse(x)) = Pi^T (fp16(||x||) * c[idx]): the residual is taken in
  the original space against what the cache actually stores;
* sign bit = 1 when (S r)_i >= 0;
* a zero vector gets idx = L/2 on every coordinate, both scales 0 and all sign
  bits 1 (the rules above with 0/0 read as 0).
"""
from __future__ import annotations

import numpy as np

from .fp16 import fp16_round


def _as64(a):
    return np.asarray(a, dtype=np.float64)


def _cells(u, boundaries):
    """idx = #{k : u >= t_k}, one comparison per threshold."""
    idx = np.zeros(u.shape, dtype=np.int64)
    for t in boundaries:
        idx += (u >= t)
    return idx


def _stage2(x, z_hat, rot, proj, sketch):
    """Residual, its norm and its sign sketch, given the stored MSE reconstruction."""
    x_mse = z_hat @ rot                 # row form of Pi^T z_hat
    r = x - x_mse                       # r = x - DEQUANT_mse(Q_mse(x))
    rho = np.sqrt(np.sum(r * r, axis=1))
    out = {"residual": r, "rho": rho}
    if sketch:
        rho16, rho_bits, rho_over = fp16_round(rho)
        p = r @ proj.T                  # S r for every vector
        out.update(rho16=rho16, rho_bits=rho_bits, rho_overflow=rho_over, p=p, sgn=(p >= 0))
    else:                               # MSE-only: no residual scale is stored
        out.update(rho_overflow=np.zeros(rho.shape, dtype=bool))
    return out


def quantize(x, rot, proj, codebook, sketch: bool = True):
    """Quantize vectors x[N, d] (exact float64 values of the stored input).

    rot: Pi [d, d]; proj: S [m, d]; codebook: dict from build_codebook with
    sigma = 1/sqrt(d).  Returns a dict with idx[N, d], sgn[N, m] (bool),
    nu, nu16, nu_bits, rho, rho16, rho_bits, flags and diagnostics u, p.
    """
    x = _as64(x)
    rot = _as64(rot)
    proj = _as64(proj)
    n, d = x.shape
    L = codebook["levels"]
    c = _as64(codebook["centroids"])
    t = _as64(codebook["boundaries"])

    nonfinite = ~np.all(np.isfinite(x), axis=1)
    # stage 1: norm, rotation, per-coordinate Lloyd-Max cell
    nu = np.sqrt(np.sum(x * x, axis=1))
    z = x @ rot.T                       # z = Pi x for every vector
    safe = np.where(nu > 0, nu, 1.0)
    u = np.where((nu > 0)[:, None], z / safe[:, None], 0.0)
    idx = _cells(u, t)
    idx[nu == 0] = L // 2
    nu16, nu_bits, nu_over = fp16_round(nu)
    z_hat = nu16[:, None] * c[idx]      # stored MSE reconstruction, rotated frame
    out = {"idx": idx, "u": u, "z": z, "nu": nu, "nu16": nu16, "nu_bits": nu_bits}
    # stage 2: residual, sign sketch and residual norm
    out.update(_stage2(x, z_hat, rot, proj, sketch))
    out["flags"] = ((nonfinite.astype(np.uint32) * 1)
                    | ((nu_over | out["rho_overflow"]).astype(np.uint32) * 2))
    return out


def quantize_conditional(x, rot, proj, codebook, idx, nu16, sketch: bool = True):
    """Stage 2 re-run with the cell indices and stored norm imposed.

    Used when the device took a different (near-tie) decision in stage 1:
    the residual, its norm and its signs then follow from that decision.
    """
    x = _as64(x)
    c = _as64(codebook["centroids"])
    z_hat = _as64(nu16)[:, None] * c[np.asarray(idx, dtype=np.int64)]
    return _stage2(x, z_hat, _as64(rot), _as64(proj), sketch)
