"""CPU tests of libtq: exported symbols, host codebook, host precomputation, argument checks.

No kernel is launched here: every call either runs host-only code or is
rejected by argument validation before anything is enqueued.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import workloads as W
from oracle import build_codebook, build_codebook_sphere

B = pytest.importorskip("kv_cache_online_amd.binding")

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "tq.h")


def test_exports_every_declared_symbol():
    src = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(tq_[a-z_]+)\s*\(", src, re.M))
    assert declared == set(B.EXPORTED), declared ^ set(B.EXPORTED)
    for name in declared:
        assert hasattr(B.LIB, name)
        assert ctypes.cast(getattr(B.LIB, name), ctypes.c_void_p).value


@pytest.mark.parametrize("bits", [1, 2, 3])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_codebook_matches_oracle(bits, d):
    s = 1 / math.sqrt(d)
    cb = B.tq_build_codebook(bits, s)
    ref = build_codebook(bits, s)
    L = 1 << bits
    assert cb.levels == L and cb.bits_mse == bits
    np.testing.assert_allclose(np.array(cb.centroid[:L]), ref["centroids"], rtol=1e-12, atol=0)
    np.testing.assert_allclose(np.array(cb.boundary[:L - 1]), ref["boundaries"], rtol=0, atol=1e-12 * s)
    assert abs(cb.mse - ref["mse"]) <= 1e-12 * ref["mse"]
    assert np.all(np.array(cb.centroid_f32[:L]) == ref["centroids"].astype(np.float32))


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_walsh_expansion_reproduces_codebook(bits):
    cb = B.tq_build_codebook(bits, 1 / math.sqrt(128))
    L = 1 << bits
    for i in range(L):
        v = 0.0
        for S in range(L):
            sg = 1.0
            for p in range(bits):
                if S >> p & 1:
                    sg *= 1.0 if (i >> p) & 1 else -1.0
            v += cb.walsh[S] * sg
        assert abs(v - cb.centroid[i]) < 1e-16
    for S in range(L):
        if bin(S).count("1") % 2 == 0:
            assert cb.walsh[S] == 0.0


def test_codebook_argument_errors():
    cb = B.tq_codebook()
    for bits, sig in ((0, 0.1), (4, 0.1), (2, 0.0), (2, -1.0), (2, float("nan"))):
        assert B.LIB.tq_build_codebook(bits, sig, ctypes.byref(cb)) == B.TQ_ERR_INVALID_ARG
    assert B.LIB.tq_build_codebook(2, 0.1, None) == B.TQ_ERR_INVALID_ARG


@pytest.mark.parametrize("bits", [1, 2, 3])
@pytest.mark.parametrize("d", [3, 8, 64, 128, 256])
def test_sphere_codebook_matches_oracle(bits, d):
    s = 1 / math.sqrt(d)
    cb = B.tq_build_codebook_sphere(bits, d)
    ref = build_codebook_sphere(bits, d)
    L = 1 << bits
    assert cb.levels == L and cb.bits_mse == bits and abs(cb.sigma - s) < 1e-16
    # both stop once a step moves the centroids by <= 1e-13 sigma, from different
    # CDF code; the iteration contracts linearly (rate near 0.95 at 3 bits), so
    # each can sit ~20 steps' worth from the fixed point: 1e-10 sigma, still
    # about 1e-3 of an fp32 ulp of the values
    np.testing.assert_allclose(np.array(cb.centroid[:L]), ref["centroids"], rtol=0, atol=1e-10 * s)
    np.testing.assert_allclose(np.array(cb.boundary[:L - 1]), ref["boundaries"], rtol=0, atol=1e-10 * s)
    assert abs(cb.mse - ref["mse"]) <= 1e-10 * ref["mse"]
    c = np.array(cb.centroid[:L])
    assert np.all(c == -c[::-1])
    # Walsh form of this codebook as well
    for i in range(L):
        v = 0.0
        for S in range(L):
            sg = 1.0
            for p in range(bits):
                if S >> p & 1:
                    sg *= 1.0 if (i >> p) & 1 else -1.0
            v += cb.walsh[S] * sg
        assert abs(v - cb.centroid[i]) <= 4 * np.spacing(abs(cb.centroid[i]))  # summation rounding only


def test_sphere_codebook_argument_errors():
    cb = B.tq_codebook()
    for bits, d in ((0, 128), (4, 128), (2, 2), (2, 0), (2, -5)):
        assert B.LIB.tq_build_codebook_sphere(bits, d, ctypes.byref(cb)) == B.TQ_ERR_INVALID_ARG
    assert B.LIB.tq_build_codebook_sphere(2, 128, None) == B.TQ_ERR_INVALID_ARG


def _bf16(v):
    u = (np.asarray(v, np.uint16).astype(np.uint32) << 16)
    return u.view(np.float32).astype(np.float64)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_prepare_blob(d):
    wid = 5 if d == 256 else 2
    P = W.rotation(d, wid)
    S = W.sketch(d, d, wid)
    blob = np.zeros(B.tq_prepare_bytes(d, d), dtype=np.uint8)
    B.tq_prepare(P, S, d, d, blob)
    hdr = blob[:16].view(np.uint32)
    assert list(hdr) == [0x31505154, 1, d, d]
    off = 256
    def take(nbytes, dtype, shape):
        nonlocal off
        a = blob[off:off + nbytes].view(dtype).reshape(shape)
        off = (off + nbytes + 255) // 256 * 256
        return a
    rotT = take(d * d * 4, np.float32, (d, d))
    stT = take(d * d * 4, np.float32, (d, d))
    projT = take(d * d * 4, np.float32, (d, d))
    rot_hml = take(3 * d * d * 2, np.uint16, (3, d, d))
    st_hml = take(3 * d * d * 2, np.uint16, (3, d, d))
    stnorm = take(d * 4, np.float32, (d,))
    assert off == len(blob)
    np.testing.assert_array_equal(rotT, P.T)
    np.testing.assert_array_equal(projT, S.T)
    st = S.astype(np.float64) @ P.astype(np.float64).T
    np.testing.assert_array_equal(stT, st.T.astype(np.float32))
    # hi + mid + lo reproduces the fp32 value exactly
    np.testing.assert_array_equal(_bf16(rot_hml[0]) + _bf16(rot_hml[1]) + _bf16(rot_hml[2]), P.astype(np.float64))
    np.testing.assert_array_equal(_bf16(st_hml[0]) + _bf16(st_hml[1]) + _bf16(st_hml[2]),
                                  st.astype(np.float32).astype(np.float64))
    np.testing.assert_allclose(stnorm, np.linalg.norm(st.astype(np.float32).astype(np.float64), axis=1), rtol=1e-6)


def test_prepare_errors():
    P = np.eye(128, dtype=np.float32)
    blob = np.zeros(B.tq_prepare_bytes(128, 128), np.uint8)
    assert B.tq_prepare_bytes(96, 96) == 0 and B.tq_prepare_bytes(128, 64) == 0
    assert B.LIB.tq_prepare(None, P.ctypes.data, 128, 128, blob.ctypes.data) == B.TQ_ERR_INVALID_ARG
    assert B.LIB.tq_prepare(P.ctypes.data, P.ctypes.data, 128, 64, blob.ctypes.data) == B.TQ_ERR_INVALID_ARG
    assert B.LIB.tq_prepare(P.ctypes.data, P.ctypes.data, 96, 96, blob.ctypes.data) == B.TQ_ERR_UNSUPPORTED


# ----------------------------------------------------- argument validation ---
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def _cfg(d=128, hkv=8, hq=32, kb=3, vb=3):
    return B.make_config(d, hkv, hq, FAKE, FAKE, FAKE, B.make_spec(kb, d), B.make_spec(vb, d))


def _cache(layout, cap=1024):
    return B.make_cache(FAKE, FAKE, FAKE, cap, layout)


def _q(cfg, **kw):
    args = dict(k=FAKE, v=FAKE, dt=B.TQ_BF16, batch=1, n_new=4, dst=FAKE,
                kc=_cache(B.TQ_LAYOUT_TOKEN_MAJOR), vc=_cache(B.TQ_LAYOUT_BLOCK32))
    args.update(kw)
    return B.LIB.tq_quantize_kv(ctypes.byref(cfg) if cfg is not None else None, args["k"], args["v"],
                                args["dt"], args["batch"], args["n_new"], args["dst"],
                                ctypes.byref(args["kc"]) if args["kc"] is not None else None,
                                ctypes.byref(args["vc"]) if args["vc"] is not None else None,
                                None, None, None)


def test_quantize_validation():
    cfg = _cfg()
    assert _q(None) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, batch=-1) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, batch=0) == B.TQ_OK                     # nothing to do, nothing enqueued
    assert _q(cfg, n_new=0) == B.TQ_OK
    assert _q(cfg, dt=7) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, k=None, v=None) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, k=FAKE + 4) == B.TQ_ERR_INVALID_ARG      # misaligned
    assert _q(cfg, dst=None) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, kc=None) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, kc=_cache(B.TQ_LAYOUT_TOKEN_MAJOR, cap=1000)) == B.TQ_ERR_INVALID_ARG
    assert _q(cfg, vc=_cache(5)) == B.TQ_ERR_INVALID_ARG
    bad = _cfg(); bad.m = 64
    assert _q(bad) == B.TQ_ERR_INVALID_ARG
    bad = _cfg(d=96)
    assert _q(bad) == B.TQ_ERR_UNSUPPORTED
    bad = _cfg(); bad.n_q_heads = 30
    assert _q(bad) == B.TQ_ERR_INVALID_ARG
    bad = _cfg(); bad.k.bits_mse = 4
    assert _q(bad) == B.TQ_ERR_INVALID_ARG
    bad = _cfg(); bad.rot = None
    assert _q(bad) == B.TQ_ERR_INVALID_ARG


def _dec(cfg, ws_bytes=None, **kw):
    args = dict(q=FAKE, dt=B.TQ_BF16, batch=2, start=FAKE, lens=FAKE, max_len=4096,
                kc=_cache(B.TQ_LAYOUT_TOKEN_MAJOR, 8192), vc=_cache(B.TQ_LAYOUT_BLOCK32, 8192),
                scale=0.0, out=FAKE, ws=FAKE)
    args.update(kw)
    need = B.LIB.tq_decode_workspace_bytes(ctypes.byref(cfg), args["batch"], args["max_len"])
    return B.LIB.tq_decode_attention(ctypes.byref(cfg), args["q"], args["dt"], args["batch"], args["start"],
                                     args["lens"], args["max_len"], ctypes.byref(args["kc"]),
                                     ctypes.byref(args["vc"]), args["scale"], args["out"], None,
                                     args["ws"], need - 1 if ws_bytes is None else ws_bytes, None)


def test_decode_validation():
    cfg = _cfg()
    assert _dec(cfg) == B.TQ_ERR_WORKSPACE
    assert _dec(cfg, batch=0) == B.TQ_OK
    assert _dec(cfg, q=None, ws_bytes=1 << 30) == B.TQ_ERR_INVALID_ARG
    assert _dec(cfg, out=FAKE + 8, ws_bytes=1 << 30) == B.TQ_ERR_INVALID_ARG
    assert _dec(cfg, scale=float("nan"), ws_bytes=1 << 30) == B.TQ_ERR_INVALID_ARG
    assert _dec(cfg, kc=_cache(B.TQ_LAYOUT_BLOCK32, 8192), ws_bytes=1 << 30) == B.TQ_ERR_UNSUPPORTED
    bad = _cfg(hq=136)   # G = 17: more query heads per kv head than the kernels take
    assert _dec(bad, ws_bytes=1 << 30) == B.TQ_ERR_UNSUPPORTED


def _score(cfg, ws_bytes=None, **kw):
    args = dict(q=FAKE, dt=B.TQ_BF16, n_q=16, kc=_cache(B.TQ_LAYOUT_TOKEN_MAJOR, 8192), kv_head=3, start=100,
                n=1000, scores=FAKE, ws=FAKE)
    args.update(kw)
    need = B.LIB.tq_score_workspace_bytes(ctypes.byref(cfg), args["n_q"], args["n"])
    return B.LIB.tq_score_keys(ctypes.byref(cfg), args["q"], args["dt"], args["n_q"], ctypes.byref(args["kc"]),
                               args["kv_head"], args["start"], args["n"], args["scores"], None, args["ws"],
                               need - 1 if ws_bytes is None else ws_bytes, None)


def test_score_validation():
    """tq_score_keys rejects bad arguments before anything is enqueued."""
    cfg = _cfg()
    big = 1 << 30
    assert _score(cfg) == B.TQ_ERR_WORKSPACE
    assert _score(cfg, n=0, ws_bytes=big) == B.TQ_OK                     # nothing to score
    for n_q in (0, 12, -8):                                              # a positive multiple of 8
        assert _score(cfg, n_q=n_q, ws_bytes=big) == B.TQ_ERR_INVALID_ARG
    assert _score(cfg, dt=7, ws_bytes=big) == B.TQ_ERR_INVALID_ARG
    assert _score(cfg, kv_head=8, ws_bytes=big) == B.TQ_ERR_INVALID_ARG  # 8 kv heads
    assert _score(cfg, kv_head=-1, ws_bytes=big) == B.TQ_ERR_INVALID_ARG
    assert _score(cfg, start=-1, ws_bytes=big) == B.TQ_ERR_INVALID_ARG
    assert _score(cfg, start=8000, n=193, ws_bytes=big) == B.TQ_ERR_INVALID_ARG  # past the capacity
    assert _score(cfg, q=None, ws_bytes=big) == B.TQ_ERR_INVALID_ARG
    assert _score(cfg, q=FAKE + 4, ws_bytes=big) == B.TQ_ERR_INVALID_ARG  # misaligned
    assert _score(cfg, scores=FAKE + 2, ws_bytes=big) == B.TQ_ERR_INVALID_ARG
    assert _score(cfg, kc=_cache(B.TQ_LAYOUT_BLOCK32, 8192), ws_bytes=big) == B.TQ_ERR_UNSUPPORTED
    assert _score(_cfg(d=64), ws_bytes=big) == B.TQ_ERR_UNSUPPORTED
    asym = _cfg()
    c = asym.k.cb
    for i in range(c.levels):                 # shift the codebook: still ordered, no longer odd
        c.centroid[i] += 1e-3
        c.centroid_f32[i] += 1e-3
    for i in range(c.levels - 1):
        c.boundary[i] += 1e-3
        c.boundary_f32[i] += 1e-3
    assert _score(asym, ws_bytes=big) == B.TQ_ERR_UNSUPPORTED
    assert B.LIB.tq_score_workspace_bytes(ctypes.byref(cfg), 12, 1000) == 0
    a = B.LIB.tq_score_workspace_bytes(ctypes.byref(cfg), 8, 1000)
    b = B.LIB.tq_score_workspace_bytes(ctypes.byref(cfg), 64, 1 << 20)
    assert 0 < a <= b


def test_workspace_plan_monotone():
    cfg = _cfg()
    a = B.tq_decode_workspace_bytes(cfg, 1, 1024)
    b = B.tq_decode_workspace_bytes(cfg, 1, 32768)
    c = B.tq_decode_workspace_bytes(cfg, 4, 131072)
    assert 0 < a <= b <= c
    assert B.tq_decode_workspace_bytes(cfg, 1, 0) > 0


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5):
        assert B.tq_status_string(s) and B.tq_status_string(s) != "unknown status"
