"""Statistical pins for the sign sketch (QJL stage) of the oracle.

ast-softpro.ru, "Технология TurboQuant и её применение с локальными LLM",
section 1.2, stage 2: the residual is projected by a random Gaussian S, only
sign(S r) is kept, and ||r||_2 is the reconstruction scale.  The estimate of
<q, r> built from those must be unbiased over draws of S; its variance has the
closed form [(pi/2) ||r||^2 ||q||^2 - <q, r>^2] / m.
"""
import math

import numpy as np
import pytest

import workloads as W
from oracle import build_codebook, quantize, dequantize


def test_gaussian_sign_expectation():
    """E[s sign(s.r)] = sqrt(2/pi) r / ||r|| for s ~ N(0, I)."""
    rng = np.random.default_rng(7)
    d = 16
    r = rng.standard_normal(d)
    s = rng.standard_normal((400000, d))
    est = (s * np.sign(s @ r)[:, None]).mean(0)
    want = math.sqrt(2 / math.pi) * r / np.linalg.norm(r)
    se = 1.0 / math.sqrt(len(s))
    assert np.max(np.abs(est - want)) < 5 * se


@pytest.fixture(scope="module")
def draws():
    w = W.WORKLOADS[1]
    d = w.d
    P = W.rotation(d, 1)
    cb = build_codebook(w.bits_mse, 1 / math.sqrt(d))
    x = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=3), w.dtype)       # three key vectors
    qv = W.to_f64(W.queries(w)[0, :3], w.dtype)                      # three queries
    est = np.zeros((1000, 3))
    r = rho = rho16 = None
    for seed in range(1000):
        S = np.random.default_rng([99, seed]).standard_normal((d, d))
        q = quantize(x, P, S, cb)
        x_mse = dequantize(q["idx"], None, q["nu16"], None, P, S, cb)
        x_hat = dequantize(q["idx"], q["sgn"], q["nu16"], q["rho16"], P, S, cb)
        r_hat = x_hat - x_mse
        est[seed] = np.sum(qv * r_hat, axis=1)
        r, rho, rho16 = q["residual"], q["rho"], q["rho16"]
    return dict(est=est, r=r, q=qv, rho=rho, rho16=rho16, m=d)


def test_unbiased_within_3_standard_errors(draws):
    est, r, qv = draws["est"], draws["r"], draws["q"]
    true = np.sum(qv * r, axis=1)
    mean = est.mean(0)
    se = est.std(0, ddof=1) / math.sqrt(len(est))
    assert np.all(np.abs(mean - true) <= 3 * se), (mean, true, se)
    # the stored fp16 residual norm scales the estimate by rho16 / rho exactly
    adj = mean * draws["rho"] / draws["rho16"]
    assert np.all(np.abs(adj - true) <= 3 * se)


def test_variance_closed_form(draws):
    est, r, qv, m = draws["est"], draws["r"], draws["q"], draws["m"]
    scale = (draws["rho16"] / draws["rho"]) ** 2
    var_cf = ((math.pi / 2) * np.sum(r * r, 1) * np.sum(qv * qv, 1) - np.sum(qv * r, 1) ** 2) / m * scale
    var = est.var(0, ddof=1)
    np.testing.assert_allclose(var, var_cf, rtol=0.15)
