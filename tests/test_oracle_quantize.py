"""Pins for the oracle's quantizer: rotation, cell rule, norms, residual, fp16 scales."""
import itertools
import math

import numpy as np
import pytest

import workloads as W
from oracle import build_codebook, fp16_round, quantize, quantize_conditional, dequantize


def _cb(bits, d):
    return build_codebook(bits, 1 / math.sqrt(d))


# ------------------------------------------------------------- rotation ---
@pytest.mark.parametrize("wid", [1, 2, 3, 4, 5])
def test_rotation_orthogonal(wid):
    w = W.WORKLOADS[wid]
    P = W.rotation(w.d, wid).astype(np.float64)
    err = np.max(np.abs(P.T @ P - np.eye(w.d)))
    assert err < 1e-5
    assert np.max(np.abs(P @ P.T - np.eye(w.d))) < 1e-5


def test_sketch_moments():
    S = W.sketch(256, 256, 5).astype(np.float64)
    assert abs(S.mean()) < 0.01 and abs(S.var() - 1) < 0.02


# ------------------------------------------------------------ cell rule ---
def test_nearest_centroid_brute_force_d4():
    """At d = 4, the per-coordinate rule is the exhaustive argmin over all L^4 code vectors."""
    d = 4
    rng = np.random.default_rng(11)
    P = W.rotation(d, 101).astype(np.float64)
    S = rng.standard_normal((d, d))
    for bits in (1, 2, 3):
        cb = _cb(bits, d)
        c = cb["centroids"]
        codes = np.array(list(itertools.product(range(cb["levels"]), repeat=d)))   # [L^4, 4]
        cand = c[codes]                                                            # [L^4, 4]
        x = rng.standard_normal((10000, d))
        q = quantize(x, P, S, cb)
        dist = ((q["u"][:, None, :] - cand[None, :, :]) ** 2).sum(-1)               # [N, L^4]
        best = codes[np.argmin(dist, axis=1)]
        np.testing.assert_array_equal(q["idx"], best)


def test_cell_rule_on_and_around_midpoints():
    """The oracle's own cell rule at exact ties: u exactly on a threshold t_k goes to the
    upper cell k + 1 (idx = #{k : u >= t_k}); one ulp below stays in cell k, one ulp
    above goes to k + 1.  Checked on the oracle's cell function itself, for every
    threshold of every width, not on a library search."""
    from oracle.quantize import _cells
    for d in (4, 128, 256):
        for bits in (1, 2, 3):
            cb = _cb(bits, d)
            t = np.asarray(cb["boundaries"], np.float64)
            for k, tk in enumerate(t):
                u = np.array([tk, np.nextafter(tk, -np.inf), np.nextafter(tk, np.inf)])
                np.testing.assert_array_equal(_cells(u, t), [k + 1, k, k + 1])
            # 0 is the middle threshold of every symmetric codebook: a tie there takes L/2
            L = cb["levels"]
            assert t[L // 2 - 1] == 0.0
            np.testing.assert_array_equal(_cells(np.array([0.0, -0.0]), t), [L // 2, L // 2])


def test_cell_rule_ties_through_quantize():
    """Ties reached through the whole quantizer.  With the identity rotation, x = e_0
    has u = (1, 0, 0, 0): three coordinates sit exactly on the middle threshold 0 and
    must take the upper cell L/2.  The smallest subnormal +-s put u = +-s, one ulp on
    either side of that threshold: cells L/2 and L/2 - 1.  A scale of x by a power of
    two leaves u exactly unchanged, so 4 e_0 gives the same cells."""
    d = 4
    tiny = np.nextafter(0.0, 1.0)
    for bits in (1, 2, 3):
        cb = _cb(bits, d)
        L = cb["levels"]
        x = np.array([[1.0, 0.0, 0.0, 0.0],
                      [4.0, 0.0, -0.0, 0.0],
                      [1.0, tiny, -tiny, 0.0]])
        q = quantize(x, np.eye(d), np.eye(d), cb)
        top = int(np.sum(1.0 >= np.asarray(cb["boundaries"])))      # u = 1 is above every threshold
        assert top == L - 1
        np.testing.assert_array_equal(q["idx"][0], [L - 1, L // 2, L // 2, L // 2])
        np.testing.assert_array_equal(q["idx"][1], [L - 1, L // 2, L // 2, L // 2])
        np.testing.assert_array_equal(q["idx"][2], [L - 1, L // 2, L // 2 - 1, L // 2])


def test_cell_rule_identity_rotation_is_sorted_search():
    """Identity rotation: cells reduce to the scalar quantizer on x / ||x||, i.e. a
    right-sided sorted search of the thresholds (random data, no ties)."""
    d = 4
    for bits in (1, 2, 3):
        cb = _cb(bits, d)
        t = cb["boundaries"]
        rng = np.random.default_rng(5)
        x = rng.standard_normal((5000, d))
        q = quantize(x, np.eye(d), np.eye(d), cb)
        u = x / np.linalg.norm(x, axis=1, keepdims=True)
        np.testing.assert_array_equal(q["idx"], np.searchsorted(t, u, side="right"))


def test_zero_vector():
    d = 8
    cb = _cb(2, d)
    P = W.rotation(d, 102)
    S = np.random.default_rng(1).standard_normal((d, d))
    q = quantize(np.zeros((1, d)), P, S, cb)
    assert np.all(q["idx"] == cb["levels"] // 2)
    assert q["nu"][0] == 0 and q["rho"][0] == 0 and q["nu_bits"][0] == 0 and q["rho_bits"][0] == 0
    assert np.all(q["sgn"])
    assert np.all(dequantize(q["idx"], q["sgn"], q["nu16"], q["rho16"], P, S, cb) == 0)


# ----------------------------------------------------- norms, residual ---
def test_norm_and_residual_consistency():
    w = W.WORKLOADS[1]
    P = W.rotation(w.d, 1)
    S = W.sketch(w.m, w.d, 1)
    cb = _cb(w.bits_mse, w.d)
    x = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=256), w.dtype)
    q = quantize(x, P, S, cb)
    np.testing.assert_allclose(q["nu"], np.linalg.norm(x, axis=1), rtol=1e-14)
    # the residual is x minus the stored MSE reconstruction (the MSE-only decode)
    x_mse = dequantize(q["idx"], None, q["nu16"], None, P, S, cb)
    np.testing.assert_allclose(q["residual"], x - x_mse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(q["rho"], np.linalg.norm(x - x_mse, axis=1), rtol=1e-13)
    # the same norm seen in the rotated frame: ||Pi x - nu16 c[idx]|| (Pi orthogonal)
    z_hat = q["nu16"][:, None] * cb["centroids"][q["idx"]]
    rot_frame = np.linalg.norm(x @ P.astype(np.float64).T - z_hat, axis=1)
    np.testing.assert_allclose(q["rho"], rot_frame, rtol=1e-6)
    # the sketch is of that residual
    np.testing.assert_allclose(q["p"], q["residual"] @ S.astype(np.float64).T, rtol=1e-12, atol=1e-12)
    assert np.array_equal(q["sgn"], q["p"] >= 0)


def test_conditional_rerun_matches():
    w = W.WORKLOADS[1]
    P, S = W.rotation(w.d, 1), W.sketch(w.m, w.d, 1)
    cb = _cb(w.bits_mse, w.d)
    x = W.to_f64(W.kv_chunk(w, 1, 0, 0, n_tokens=64), w.dtype)
    q = quantize(x, P, S, cb)
    c = quantize_conditional(x, P, S, cb, q["idx"], q["nu16"])
    np.testing.assert_array_equal(c["sgn"], q["sgn"])
    np.testing.assert_array_equal(c["rho"], q["rho"])
    # a flipped cell changes the residual and hence the stored residual norm
    idx2 = q["idx"].copy()
    idx2[0, 0] = (idx2[0, 0] + 1) % cb["levels"]
    c2 = quantize_conditional(x, P, S, cb, idx2, q["nu16"])
    assert c2["rho"][0] != q["rho"][0]


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_distortion_within_pages_bound(bits):
    """MSE of the rotated unit vector vs its codebook value, against 2.7 * 4^-b'.

    kiosknews.app, "3 бита вместо 16…", section "Как работает TurboQuant": the
    distortion is provably within about 2.7x of the information-theoretic
    minimum 4^-b' for unit vectors.  It should also sit near the Gaussian
    Lloyd-Max distortion per coordinate times d.
    """
    d = 128
    rng = np.random.default_rng(3)
    P = W.rotation(d, 103)
    cb = _cb(bits, d)
    x = rng.standard_normal((4000, d)) * np.exp(rng.uniform(-3, 3, (4000, 1)))
    q = quantize(x, P, np.eye(d), cb)
    u_hat = cb["centroids"][q["idx"]]
    dist = np.mean(np.sum((q["u"] - u_hat) ** 2, axis=1))
    assert dist <= 2.7 * 4.0 ** (-bits)
    assert abs(dist - cb["mse"] * d) < 0.05 * cb["mse"] * d


def test_mse_only_mode():
    w = W.WORKLOADS[1]
    P, S = W.rotation(w.d, 1), W.sketch(w.m, w.d, 1)
    cb = _cb(3, w.d)
    x = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=32), w.dtype)
    q = quantize(x, P, S, cb, sketch=False)
    assert "sgn" not in q and "rho_bits" not in q
    full = quantize(x, P, S, cb)
    np.testing.assert_array_equal(q["idx"], full["idx"])


# ------------------------------------------------------------- scales ---
def test_fp16_rounding_cases():
    one = 1.0
    ulp = 2.0 ** -10
    cases = [
        (one + ulp / 2, one),                            # tie -> even (1.0)
        (one + ulp / 2 + 2.0 ** -30, one + ulp),         # just above the tie -> up
        (one + 3 * ulp / 2, one + 2 * ulp),              # tie -> even (mantissa 2)
        (65504.0, 65504.0),
        (2.0 ** -24, 2.0 ** -24), (2.0 ** -25, 0.0),     # subnormal tie -> even (0)
        (3 * 2.0 ** -26, 2.0 ** -24),
    ]
    for x, want in cases:
        v, bits, over = fp16_round(np.array([x]))
        assert v[0] == want, (x, v[0], want)
        assert not over[0]
    v, bits, over = fp16_round(np.array([65504.5, 65519.0, 1e6]))
    assert np.all(v == 65504.0) and np.all(over) and np.all(bits == 0x7BFF)


def test_flags():
    d = 8
    cb = _cb(2, d)
    P = W.rotation(d, 104)
    S = np.eye(d)
    x = np.ones((3, d))
    x[1, 2] = np.nan
    x[2] *= 1e5                                       # ||x|| > 65504
    q = quantize(x, P, S, cb)
    assert q["flags"][0] == 0
    assert q["flags"][1] & 1
    assert q["flags"][2] & 2
