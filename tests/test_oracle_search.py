"""Pins for the oracle's search scores (oracle.score_keys).

ast-softpro.ru, "Технология TurboQuant и её применение с локальными LLM",
section 6.4 and FAQ: the compressed vectors serve as a vector-search index; a
score is the inner product with the encoded vector (section 1.2's estimator).
Pinned by: over draws of S the scores are unbiased for the true <q, x>; with
the sketch off they equal the rotated-frame inner product <Pi q, nu~ c[idx]>;
they are linear in the query; and a softmax over them reproduces the
attention oracle (itself pinned against torch's scaled dot-product attention).
"""
import math

import numpy as np

import workloads as W
from oracle import attention, build_codebook, dequantize, quantize, score_keys


def _setup(n_tokens):
    w = W.WORKLOADS[1]
    d = w.d
    P, S = W.rotation(d, 1), W.sketch(d, d, 1)
    cb = build_codebook(w.bits_mse, 1 / math.sqrt(d))
    x = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=n_tokens), w.dtype)
    return w, d, P, S, cb, x


def test_unbiased_over_sketch_draws():
    """Mean over 600 draws of S of the score of a quantized vector equals <q, x>
    within 3 standard errors (rho unrounded, so the target is exactly <q, x>)."""
    w, d, P, _, cb, x = _setup(2)
    qv = W.to_f64(W.queries(w)[0, :2], w.dtype)
    est = np.zeros((600, 2, 2))
    for seed in range(600):
        S = np.random.default_rng([123, seed]).standard_normal((d, d))
        o = quantize(x, P, S, cb)
        est[seed] = score_keys(qv, o["idx"], o["sgn"], o["nu16"], o["rho"], P, S, cb)
    true = qv @ x.T
    mean = est.mean(0)
    se = est.std(0, ddof=1) / math.sqrt(len(est))
    assert np.all(np.abs(mean - true) <= 3 * se), (mean, true, se)


def test_sketch_off_is_the_rotated_frame_product():
    w, d, P, S, cb, x = _setup(7)
    o = quantize(x, P, S, cb, sketch=False)
    q = np.random.default_rng(4).standard_normal((3, d))
    got = score_keys(q, o["idx"], None, o["nu16"], None, P, S, cb)
    zhat = o["nu16"][:, None] * np.asarray(cb["centroids"])[o["idx"]]
    want = (q @ P.T) @ zhat.T            # <Pi q, z_hat>, no inverse rotation
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_linear_in_the_query():
    w, d, P, S, cb, x = _setup(5)
    o = quantize(x, P, S, cb)
    rng = np.random.default_rng(3)
    q1, q2 = rng.standard_normal((2, d)), rng.standard_normal((2, d))
    f = lambda q: score_keys(q, o["idx"], o["sgn"], o["nu16"], o["rho16"], P, S, cb)
    np.testing.assert_allclose(f(2.5 * q1 - 0.75 * q2), 2.5 * f(q1) - 0.75 * f(q2), rtol=1e-12, atol=1e-12)


def test_softmax_of_scores_is_the_attention_oracle():
    w, d, P, S, cb, x = _setup(40)
    o = quantize(x, P, S, cb)
    k_hat = dequantize(o["idx"], o["sgn"], o["nu16"], o["rho16"], P, S, cb)
    v = np.random.default_rng(8).standard_normal((40, d))
    q = W.to_f64(W.queries(w)[0, :4], w.dtype)
    s = score_keys(q, o["idx"], o["sgn"], o["nu16"], o["rho16"], P, S, cb) / math.sqrt(d)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    want = (p / p.sum(axis=1, keepdims=True)) @ v
    got = attention(q, k_hat[None], v[None])
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-12)
