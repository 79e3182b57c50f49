"""Decode attention over reconstructed keys and values (oracle; test infrastructure only).

The pages say decode attention reads the compressed cache (the speed-up comes
from moving less data: ast-softpro.ru, "Технология TurboQuant и её применение с
локальными LLM", section 1.3; kiosknews.app, "3 бита вместо 16…", section
"8x и «zero loss»") but do not restate attention itself.  Reading: standard
scaled dot-product attention for one new query per (sequence, query head):
s_t = <q, k_hat_t> * scale (scale = 1/sqrt(d) by default), softmax over all
cached tokens of the sequence (max-subtracted), output sum_t p_t v_hat_t.
Grouped-query mapping: query head h reads kv head h // G with G = H_q / H_kv.
"""
from __future__ import annotations

import numpy as np


def attention(q, k_hat, v_hat, scale=None):
    """q[H_q, d]; k_hat, v_hat [H_kv, T, d] (one sequence) -> out[H_q, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    hq, d = q.shape
    hkv = k_hat.shape[0]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((hq, d))
    for h in range(hq):
        kv = h // g
        s = (k_hat[kv] @ q[h]) * scale          # one score per cached token
        p = np.exp(s - np.max(s))
        p = p / np.sum(p)
        out[h] = p @ v_hat[kv]
    return out
