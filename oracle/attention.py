"""Decode attention over reconstructed keys and values (oracle; test infrastructure only).

The pages say decode attention reads the compressed cache (the speed-up comes
from moving less data: ast-softpro.ru, "Технология TurboQuant и её применение с
локальными LLM", section 1.3; kiosknews.app, "3 бита вместо 16…", section
"8x и «zero loss»") but do not restate attention itself.  Reading: standard
scaled dot-product attention for one new query per (sequence, query head):
s_t = <q, k_hat_t> * scale (scale = 1/sqrt(d) by default), softmax over all
cached tokens of the sequence (max-subtracted), output sum_t p_t v_hat_t.
Grouped-query mapping: query head h reads kv head h // G with G = H_q / H_kv.

Sparse V (kiosknews.app, "3 бита вместо 16: разбираем TurboQuant и когда его
реально стоит включать", section "Что работает прямо сейчас и как попробовать",
llama.cpp paragraph): decode skips the positions whose attention weight is low.
The page gives no threshold rule; reading taken: with M the largest score of the
row, position t is skipped when its weight relative to the largest one,
exp(s_t - M), is below a caller's tau in [0, 1] (s_t < M + ln tau); the softmax
normalizer still runs over every position (the weights are what they are; only
the skipped positions' values are left out of the sum), so the output is
sum over kept t of p_t v_hat_t.  tau = 0 skips nothing.
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


def attention_sparse_v(q, k_hat, v_hat, tau, scale=None):
    """Sparse V decode attention: like attention(), but the value of position t
    is left out of the weighted sum when exp(s_t - M) < tau, M the row's largest
    score; the weights keep the normalizer over every position.  Returns
    out[H_q, d] float64 and the kept mask [H_q, T] (bool)."""
    q = np.asarray(q, dtype=np.float64)
    k_hat = np.asarray(k_hat, dtype=np.float64)
    v_hat = np.asarray(v_hat, dtype=np.float64)
    hq, d = q.shape
    hkv, T = k_hat.shape[0], k_hat.shape[1]
    if hq % hkv:
        raise ValueError("query heads must be a multiple of kv heads")
    if not 0.0 <= tau <= 1.0:
        raise ValueError("tau must lie in [0, 1]")
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((hq, d))
    kept = np.zeros((hq, T), dtype=bool)
    for h in range(hq):
        kv = h // g
        s = (k_hat[kv] @ q[h]) * scale
        m = np.max(s)
        w = np.exp(s - m)                       # weight relative to the largest, in (0, 1]
        p = w / np.sum(w)                       # softmax over every position
        keep = w >= tau
        kept[h] = keep
        out[h] = p[keep] @ v_hat[kv][keep]      # values of the kept positions only
    return out, kept
