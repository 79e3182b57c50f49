"""Pins for the oracle's Sparse V attention (values of positions whose weight
relative to the row's largest is below tau are left out; the normalizer keeps
every position).  Pinned against torch's scaled_dot_product_attention on the CPU
in float64 -- skipping a position's value is the same as zeroing that value row --
and against closed forms for tau = 0 and tau = 1."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, attention_sparse_v


def _data(seed, hq=4, hkv=2, T=300, d=16, spread=3.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((hq, d)) * spread
    k = rng.standard_normal((hkv, T, d))
    v = rng.standard_normal((hkv, T, d))
    return q, k, v


def _sdpa(q, k, v, scale):
    """torch SDPA (CPU, float64), query head h on kv head h // G."""
    hq, hkv = q.shape[0], k.shape[0]
    g = hq // hkv
    kk = torch.from_numpy(np.repeat(k, g, axis=0))[:, None]      # [hq, 1, T, d]
    vv = torch.from_numpy(np.repeat(v, g, axis=0))[:, None]
    qq = torch.from_numpy(q)[:, None, None]                       # [hq, 1, 1, d]
    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=scale)[:, 0, 0].numpy()


@pytest.mark.parametrize("tau", [1e-6, 1e-3, 0.05, 0.5])
def test_equals_sdpa_with_skipped_value_rows_zeroed(tau):
    q, k, v = _data(1)
    scale = 1 / math.sqrt(q.shape[1])
    out, kept = attention_sparse_v(q, k, v, tau, scale)
    g = q.shape[0] // k.shape[0]
    for h in range(q.shape[0]):
        # the kept set from torch's own scores: exp(s - max) >= tau
        s = (torch.from_numpy(k[h // g]) @ torch.from_numpy(q[h])) * scale
        keep = torch.exp(s - s.max()) >= tau
        np.testing.assert_array_equal(kept[h], keep.numpy())
        vz = v.copy()
        vz[h // g][~keep.numpy()] = 0.0
        ref = _sdpa(q[h:h + 1], k[h // g:h // g + 1], vz[h // g:h // g + 1], scale)[0]
        np.testing.assert_allclose(out[h], ref, rtol=0, atol=1e-12)
    assert 0 < kept.sum() < kept.size          # something was skipped, something kept


def test_tau_zero_is_plain_attention():
    q, k, v = _data(2)
    out, kept = attention_sparse_v(q, k, v, 0.0)
    assert kept.all()
    np.testing.assert_allclose(out, attention(q, k, v), rtol=0, atol=1e-13)


def test_tau_one_keeps_only_the_maximum():
    """tau = 1 keeps only the positions with the largest score; with one such
    position t*, out = v_t* / sum_t exp(s_t - s_t*)."""
    q, k, v = _data(3, hq=2, hkv=1, T=50, d=8)
    scale = 0.7
    out, kept = attention_sparse_v(q, k, v, 1.0, scale)
    for h in range(2):
        s = k[0] @ q[h] * scale
        t = int(np.argmax(s))
        assert kept[h].sum() == 1 and kept[h, t]
        np.testing.assert_allclose(out[h], v[0, t] / np.sum(np.exp(s - s[t])), rtol=1e-13)


def test_skipped_mass_bounds_the_change():
    """The change from dense attention is the skipped positions' weighted values:
    at most (skipped softmax mass) x max|v|, and each skipped weight is below tau
    times the largest one."""
    q, k, v = _data(4)
    dense = attention(q, k, v)
    for tau in (1e-4, 1e-2, 0.2):
        out, kept = attention_sparse_v(q, k, v, tau)
        g = q.shape[0] // k.shape[0]
        for h in range(q.shape[0]):
            s = k[h // g] @ q[h] / math.sqrt(q.shape[1])
            p = np.exp(s - s.max())
            p /= p.sum()
            mass = p[~kept[h]].sum()
            assert np.max(np.abs(out[h] - dense[h])) <= mass * np.abs(v[h // g]).max() + 1e-15
            assert np.all(p[~kept[h]] < tau * p.max())
