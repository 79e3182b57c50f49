"""Inner-product scores against packed vectors (oracle; test infrastructure only).

[softpro §6.4, FAQ] ast-softpro.ru, "Технология TurboQuant и её применение с
локальными LLM", section 6.4 and the FAQ: the same compression serves vector
search (RAG indexes) over any high-dimensional vectors.  The score of a query
against a compressed vector is the inner product with the vector the record
encodes, <q, x_hat>, with x_hat as in ``dequantize`` ([softpro §1.2]: the
rotated MSE part plus the sign-sketch correction that makes the estimate of
<q, x> unbiased).  Plain definition: a float64 matrix product.
"""
from __future__ import annotations

import numpy as np

from .dequant import dequantize


def score_keys(q, idx, sgn, nu16, rho16, rot, proj, codebook):
    """scores[n_q, N] = q @ x_hat^T in float64 (sgn None: sketch off)."""
    x_hat = dequantize(idx, sgn, nu16, rho16, rot, proj, codebook)
    return np.asarray(q, dtype=np.float64) @ x_hat.T
