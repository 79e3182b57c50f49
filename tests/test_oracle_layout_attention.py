"""Pins for the oracle's packing, reconstruction and attention."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import (attention, build_codebook, dequantize, pack_block32, pack_token_major,
                    quantize, record_bytes, unpack_block32, unpack_token_major)


# ------------------------------------------------------------- packing ---
def test_token_major_known_words():
    d, bits = 64, 2
    idx = np.tile(np.arange(d) % 4, (1, 1))
    sgn = (np.arange(d) < 5)[None, :]
    iw, sw, scl = pack_token_major(idx, sgn, np.array([0x3C00]), np.array([0x4000]), bits)
    assert iw.shape == (1, 2, 2) and sw.shape == (1, 2)
    assert np.all(iw[0, 0] == 0xAAAAAAAA)          # plane 0: odd coordinates
    assert np.all(iw[0, 1] == 0xCCCCCCCC)          # plane 1: coordinates with j % 4 >= 2
    assert sw[0, 0] == 0x1F and sw[0, 1] == 0
    assert list(scl[0]) == [0x3C00, 0x4000]


def test_block32_known_words():
    d, bits, n = 32, 3, 64
    idx = np.zeros((n, d), dtype=np.int64)
    idx[:, 0] = np.arange(n) % 8                   # coordinate 0 cycles through all codes
    idx[5, 7] = 7
    sgn = np.zeros((n, d), dtype=bool)
    sgn[33, 4] = True
    iw, sw, scl = pack_block32(idx, sgn, np.zeros(n, np.uint16), np.zeros(n, np.uint16), bits)
    assert iw.shape == (2, 3, d) and sw.shape == (2, d)
    assert iw[0, 0, 0] == 0xAAAAAAAA and iw[0, 1, 0] == 0xCCCCCCCC and iw[0, 2, 0] == 0xF0F0F0F0
    assert iw[0, 0, 7] == 1 << 5 and iw[0, 1, 7] == 1 << 5 and iw[0, 2, 7] == 1 << 5
    assert sw[1, 4] == 1 << 1 and np.count_nonzero(sw) == 1


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    n, d = 96, 128
    idx = rng.integers(0, 1 << bits, (n, d))
    sgn = rng.random((n, d)) < 0.5
    nb = rng.integers(0, 65535, n).astype(np.uint16)
    rb = rng.integers(0, 65535, n).astype(np.uint16)
    for pack, unpack in ((pack_token_major, unpack_token_major), (pack_block32, unpack_block32)):
        i2, s2, n2, r2 = unpack(*pack(idx, sgn, nb, rb, bits), bits)
        np.testing.assert_array_equal(i2, idx)
        np.testing.assert_array_equal(s2, sgn)
        np.testing.assert_array_equal(n2, nb)
        np.testing.assert_array_equal(r2, rb)


def test_record_sizes_match_pages_ratios():
    # kiosknews.app "3 бита вместо 16…", llama.cpp formats: turbo3 5x, turbo4 3.8x vs fp16
    assert record_bytes(128, 128, 2) == 52 and record_bytes(128, 128, 3) == 68
    assert record_bytes(256, 256, 1) == 68
    r3 = 16 / (52 * 8 / 128)
    r4 = 16 / (68 * 8 / 128)
    assert round(r3) == 5 and round(r4, 1) == 3.8
    # the same page: a 70B-class model (80 layers, 8 kv heads, d=128) at 128K in bf16 ~ 40 GB
    bf16 = 80 * 8 * 128 * 2 * 2 * 131072
    assert bf16 == 40 * 2 ** 30
    packed = 80 * 8 * 131072 * 2 * record_bytes(128, 128, 2)
    assert abs(packed / 2 ** 30 - 8.125) < 1e-9


# ------------------------------------------------------- reconstruction ---
def _setup(n=64, bits=2, d=128, seed=0):
    rng = np.random.default_rng(seed)
    P = W.rotation(d, 200 + seed)
    S = rng.standard_normal((d, d)).astype(np.float32)
    cb = build_codebook(bits, 1 / math.sqrt(d))
    x = rng.standard_normal((n, d))
    return P, S, cb, x, quantize(x, P, S, cb)


def test_dequant_special_cases():
    P, S, cb, x, q = _setup()
    mse = dequantize(q["idx"], q["sgn"], q["nu16"], np.zeros_like(q["rho16"]), P, S, cb)
    np.testing.assert_array_equal(mse, dequantize(q["idx"], None, q["nu16"], None, P, S, cb))
    a = dequantize(q["idx"], q["sgn"], q["nu16"], q["rho16"], P, S, cb)
    b = dequantize(q["idx"], q["sgn"], 2 * q["nu16"], 2 * q["rho16"], P, S, cb)
    np.testing.assert_allclose(b, 2 * a, rtol=1e-13, atol=1e-13)
    # reconstruction improves on the MSE part for inner products on average
    qv = np.random.default_rng(9).standard_normal((200, x.shape[1]))
    e_full = np.mean((qv @ (x - a).T) ** 2)
    e_mse = np.mean((qv @ (x - mse).T) ** 2)
    assert e_full < 10 * e_mse  # same order: the sign part adds variance, not bias


# ------------------------------------------------------------ attention ---
def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    hq, hkv, t, d = 8, 2, 37, 16
    q = rng.standard_normal((hq, d))
    k = rng.standard_normal((hkv, t, d)) * 2
    v = rng.standard_normal((hkv, t, d))
    out = attention(q, k, v)
    g = hq // hkv
    kt = torch.from_numpy(np.repeat(k, g, axis=0))[None]
    vt = torch.from_numpy(np.repeat(v, g, axis=0))[None]
    qt = torch.from_numpy(q)[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0, :].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(5)
    d = 16
    q = rng.standard_normal((4, d))
    v = rng.standard_normal((1, 9, d))
    # one cached token: the output is that token's value
    np.testing.assert_allclose(attention(q, rng.standard_normal((1, 1, d)), v[:, :1]),
                               np.repeat(v[0, :1], 4, 0), rtol=1e-15)
    # identical keys: the output is the mean value
    k = np.repeat(rng.standard_normal((1, 1, d)), 9, axis=1)
    np.testing.assert_allclose(attention(q, k, v), np.repeat(v[0].mean(0, keepdims=True), 4, 0), rtol=1e-12)
    # one dominant score: the output tends to that token's value
    k = rng.standard_normal((1, 9, d)) * 0.01
    k[0, 3] = q[0] * 1e3
    np.testing.assert_allclose(attention(q[:1], k, v)[0], v[0, 3], atol=1e-9)


def test_attention_gqa_mapping():
    d, t = 8, 5
    hkv, g = 3, 2
    q = np.ones((hkv * g, d))
    k = np.zeros((hkv, t, d))
    v = np.stack([np.full((t, d), float(h)) for h in range(hkv)])
    out = attention(q, k, v)
    for h in range(hkv * g):
        assert np.all(out[h] == h // g)


def test_decode_restructuring_identity():
    """Scores and outputs from rotated-frame accumulators equal attention over x_hat.

    s_t = [nu16_t <Pi q, c[idx_t]> + kappa rho16_t <S q, 2 sgn_t - 1>] / sqrt(d);
    out = [Pi^T sum_t p_t nu16_t c[idx_t] + kappa S^T sum_t p_t rho16_t (2 sgn_t - 1)] / sum_t p_t.
    This is the form the device kernels evaluate.
    """
    P, S, cb, x, qk = _setup(n=50, seed=1)
    _, _, _, y, qv = _setup(n=50, seed=2)
    P2, S2 = P, S
    qv = quantize(y, P2, S2, cb)
    d = x.shape[1]
    kappa = math.sqrt(math.pi / 2) / S.shape[0]
    k_hat = dequantize(qk["idx"], qk["sgn"], qk["nu16"], qk["rho16"], P, S, cb)
    v_hat = dequantize(qv["idx"], qv["sgn"], qv["nu16"], qv["rho16"], P, S, cb)
    q = np.random.default_rng(3).standard_normal((2, d))
    ref = attention(q, k_hat[None], v_hat[None])
    P64, S64 = P.astype(np.float64), S.astype(np.float64)
    c = cb["centroids"]
    for h in range(2):
        q_rot, q_s = P64 @ q[h], S64 @ q[h]
        s = (qk["nu16"] * (c[qk["idx"]] @ q_rot)
             + kappa * qk["rho16"] * (np.where(qk["sgn"], 1.0, -1.0) @ q_s)) / math.sqrt(d)
        p = np.exp(s - s.max())
        A = (p * qv["nu16"]) @ c[qv["idx"]]
        B = (p * qv["rho16"]) @ np.where(qv["sgn"], 1.0, -1.0)
        out = (P64.T @ A + kappa * (S64.T @ B)) / p.sum()
        np.testing.assert_allclose(out, ref[h], rtol=1e-12, atol=1e-12)
