"""ctypes binding of libtq (include/tq.h), names identical to the C entry points.

Argument marshalling only: every step of the quantize and decode paths runs in
libtq's HIP kernels.  PyTorch supplies device memory (``tensor.data_ptr()``)
and the HIP stream (``torch.cuda.current_stream().cuda_stream``).  If
libtq.so has not been built this module raises at import time: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import (POINTER, Structure, c_char_p, c_double, c_float, c_int, c_int32, c_int64,
                    c_size_t, c_void_p)

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")

TQ_OK, TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_WORKSPACE, TQ_ERR_LAUNCH, TQ_ERR_NO_CONVERGENCE = \
    0, -1, -2, -3, -4, -5
TQ_F32, TQ_BF16 = 0, 1
TQ_LAYOUT_TOKEN_MAJOR, TQ_LAYOUT_BLOCK32 = 0, 1
TQ_FLAG_NONFINITE_INPUT, TQ_FLAG_SCALE_OVERFLOW, TQ_FLAG_OUT_OF_RANGE = 1, 2, 4
TQ_MAX_LEVELS = 8

EXPORTED = ("tq_build_codebook", "tq_build_codebook_sphere", "tq_prepare_bytes", "tq_prepare", "tq_quantize_kv",
            "tq_decode_workspace_bytes", "tq_decode_attention", "tq_decode_attention_sparse_v",
            "tq_decode_attention_noalloc",
            "tq_score_workspace_bytes", "tq_score_keys", "tq_status_string")
TQ_NOALLOC_SCRATCH_BYTES = 64 << 20


class tq_codebook(Structure):
    _fields_ = [("bits_mse", c_int32), ("levels", c_int32), ("sigma", c_double),
                ("centroid", c_double * TQ_MAX_LEVELS), ("boundary", c_double * (TQ_MAX_LEVELS - 1)),
                ("centroid_f32", c_float * TQ_MAX_LEVELS),
                ("boundary_f32", c_float * (TQ_MAX_LEVELS - 1)),
                ("walsh", c_double * TQ_MAX_LEVELS), ("mse", c_double), ("iterations", c_int32)]


class tq_tensor_spec(Structure):
    _fields_ = [("bits_mse", c_int32), ("sketch", c_int32), ("cb", tq_codebook)]


class tq_config(Structure):
    _fields_ = [("d", c_int32), ("m", c_int32), ("n_kv_heads", c_int32), ("n_q_heads", c_int32),
                ("rot", c_void_p), ("proj", c_void_p), ("prep", c_void_p),
                ("k", tq_tensor_spec), ("v", tq_tensor_spec)]


class tq_cache(Structure):
    _fields_ = [("idx", c_void_p), ("sgn", c_void_p), ("scl", c_void_p),
                ("capacity", c_int64), ("layout", c_int32)]


class TQError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {tq_status_string(status)} ({status})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"libtq.so is not built ({_LIB_PATH}); run "
                          "`python kv_cache_online_amd/build.py` (needs hipcc)")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.tq_build_codebook.argtypes = [c_int32, c_double, POINTER(tq_codebook)]
    lib.tq_build_codebook.restype = c_int
    lib.tq_build_codebook_sphere.argtypes = [c_int32, c_int32, POINTER(tq_codebook)]
    lib.tq_build_codebook_sphere.restype = c_int
    lib.tq_prepare_bytes.argtypes = [c_int32, c_int32]
    lib.tq_prepare_bytes.restype = c_size_t
    lib.tq_prepare.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p]
    lib.tq_prepare.restype = c_int
    lib.tq_quantize_kv.argtypes = [POINTER(tq_config), c_void_p, c_void_p, c_int, c_int32, c_int32,
                                   c_void_p, POINTER(tq_cache), POINTER(tq_cache), c_void_p, c_void_p,
                                   c_void_p]
    lib.tq_quantize_kv.restype = c_int
    lib.tq_decode_workspace_bytes.argtypes = [POINTER(tq_config), c_int32, c_int32]
    lib.tq_decode_workspace_bytes.restype = c_size_t
    lib.tq_decode_attention.argtypes = [POINTER(tq_config), c_void_p, c_int, c_int32, c_void_p,
                                        c_void_p, c_int32, POINTER(tq_cache), POINTER(tq_cache),
                                        c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.tq_decode_attention.restype = c_int
    lib.tq_decode_attention_sparse_v.argtypes = [POINTER(tq_config), c_void_p, c_int, c_int32, c_void_p,
                                                 c_void_p, c_int32, POINTER(tq_cache), POINTER(tq_cache),
                                                 c_float, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                                 c_void_p]
    lib.tq_decode_attention_sparse_v.restype = c_int
    lib.tq_decode_attention_noalloc.argtypes = [POINTER(tq_config), c_void_p, c_int, c_int32, c_void_p,
                                                c_void_p, c_int32, POINTER(tq_cache), POINTER(tq_cache),
                                                c_float, c_void_p, c_void_p, c_void_p]
    lib.tq_decode_attention_noalloc.restype = c_int
    lib.tq_score_workspace_bytes.argtypes = [POINTER(tq_config), c_int32, c_int32]
    lib.tq_score_workspace_bytes.restype = c_size_t
    lib.tq_score_keys.argtypes = [POINTER(tq_config), c_void_p, c_int, c_int32, POINTER(tq_cache), c_int32,
                                  ctypes.c_int64, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.tq_score_keys.restype = c_int
    lib.tq_status_string.argtypes = [c_int]
    lib.tq_status_string.restype = c_char_p
    return lib


LIB = _load()
LIB_PATH = _LIB_PATH


def _ptr(t):
    """Device (or host) address of a tensor / numpy array, or None."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if hasattr(t, "ctypes"):
        return t.ctypes.data
    return int(t)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


# ------------------------------------------------------------ entry points ---
def tq_status_string(status: int) -> str:
    return LIB.tq_status_string(status).decode()


def tq_build_codebook(bits_mse: int, sigma: float) -> tq_codebook:
    cb = tq_codebook()
    st = LIB.tq_build_codebook(bits_mse, sigma, ctypes.byref(cb))
    if st != TQ_OK:
        raise TQError(st, "tq_build_codebook")
    return cb


def tq_build_codebook_sphere(bits_mse: int, d: int) -> tq_codebook:
    cb = tq_codebook()
    st = LIB.tq_build_codebook_sphere(bits_mse, d, ctypes.byref(cb))
    if st != TQ_OK:
        raise TQError(st, "tq_build_codebook_sphere")
    return cb


def tq_prepare_bytes(d: int, m: int) -> int:
    return LIB.tq_prepare_bytes(d, m)


def tq_prepare(rot_host, proj_host, d: int, m: int, blob_host) -> None:
    """rot_host, proj_host: float32 C-contiguous host arrays; blob_host: writable host buffer."""
    st = LIB.tq_prepare(_ptr(rot_host), _ptr(proj_host), d, m, _ptr(blob_host))
    if st != TQ_OK:
        raise TQError(st, "tq_prepare")


def tq_quantize_kv(cfg: tq_config, k, v, dt: int, batch: int, n_new: int, dst_token,
                   kc: tq_cache, vc: tq_cache, status=None, dbg_scales=None, stream=None) -> None:
    st = LIB.tq_quantize_kv(ctypes.byref(cfg), _ptr(k), _ptr(v), dt, batch, n_new, _ptr(dst_token),
                            ctypes.byref(kc) if kc is not None else None,
                            ctypes.byref(vc) if vc is not None else None,
                            _ptr(status), _ptr(dbg_scales), _stream(stream))
    if st != TQ_OK:
        raise TQError(st, "tq_quantize_kv")


def tq_decode_workspace_bytes(cfg: tq_config, batch: int, max_len: int) -> int:
    return LIB.tq_decode_workspace_bytes(ctypes.byref(cfg), batch, max_len)


def tq_decode_attention(cfg: tq_config, q, dt: int, batch: int, seq_start, seq_len, max_len: int,
                        kc: tq_cache, vc: tq_cache, sm_scale: float, out, status, workspace,
                        ws_bytes: int, stream=None) -> None:
    st = LIB.tq_decode_attention(ctypes.byref(cfg), _ptr(q), dt, batch, _ptr(seq_start), _ptr(seq_len),
                                 max_len, ctypes.byref(kc), ctypes.byref(vc), sm_scale, _ptr(out),
                                 _ptr(status), _ptr(workspace), ws_bytes, _stream(stream))
    if st != TQ_OK:
        raise TQError(st, "tq_decode_attention")


def tq_decode_attention_sparse_v(cfg: tq_config, q, dt: int, batch: int, seq_start, seq_len, max_len: int,
                                 kc: tq_cache, vc: tq_cache, sm_scale: float, tau: float, out, status, workspace,
                                 ws_bytes: int, stream=None) -> None:
    st = LIB.tq_decode_attention_sparse_v(ctypes.byref(cfg), _ptr(q), dt, batch, _ptr(seq_start), _ptr(seq_len),
                                          max_len, ctypes.byref(kc), ctypes.byref(vc), sm_scale, tau, _ptr(out),
                                          _ptr(status), _ptr(workspace), ws_bytes, _stream(stream))
    if st != TQ_OK:
        raise TQError(st, "tq_decode_attention_sparse_v")


def tq_decode_attention_noalloc(cfg: tq_config, q, dt: int, batch: int, seq_start, seq_len, max_len: int,
                                kc: tq_cache, vc: tq_cache, sm_scale: float, out, status, stream=None) -> None:
    st = LIB.tq_decode_attention_noalloc(ctypes.byref(cfg), _ptr(q), dt, batch, _ptr(seq_start), _ptr(seq_len),
                                         max_len, ctypes.byref(kc), ctypes.byref(vc), sm_scale, _ptr(out),
                                         _ptr(status), _stream(stream))
    if st != TQ_OK:
        raise TQError(st, "tq_decode_attention_noalloc")


def tq_score_workspace_bytes(cfg: tq_config, n_q: int, max_n: int) -> int:
    return LIB.tq_score_workspace_bytes(ctypes.byref(cfg), n_q, max_n)


def tq_score_keys(cfg: tq_config, q, dt: int, n_q: int, kc: tq_cache, kv_head: int, start: int, n: int,
                  scores, status, workspace, ws_bytes: int, stream=None) -> None:
    st = LIB.tq_score_keys(ctypes.byref(cfg), _ptr(q), dt, n_q, ctypes.byref(kc), kv_head, start, n,
                           _ptr(scores), _ptr(status), _ptr(workspace), ws_bytes, _stream(stream))
    if st != TQ_OK:
        raise TQError(st, "tq_score_keys")


# ------------------------------------------------- struct helpers (host) ---
def make_spec(bits_mse: int, d: int, sketch: int = 1, law: str = "gaussian") -> tq_tensor_spec:
    """law: "gaussian" (N(0, 1/d), tq_build_codebook) or "sphere" (exact law of a
    unit-vector coordinate, tq_build_codebook_sphere)."""
    s = tq_tensor_spec()
    s.bits_mse = bits_mse
    s.sketch = sketch
    if law == "gaussian":
        s.cb = tq_build_codebook(bits_mse, 1.0 / math.sqrt(d))
    elif law == "sphere":
        s.cb = tq_build_codebook_sphere(bits_mse, d)
    else:
        raise ValueError(f"unknown codebook law {law!r}")
    return s


def make_config(d: int, n_kv_heads: int, n_q_heads: int, rot_dev, proj_dev, prep_dev,
                k_spec: tq_tensor_spec, v_spec: tq_tensor_spec) -> tq_config:
    c = tq_config()
    c.d = d
    c.m = d
    c.n_kv_heads = n_kv_heads
    c.n_q_heads = n_q_heads
    c.rot = _ptr(rot_dev)
    c.proj = _ptr(proj_dev)
    c.prep = _ptr(prep_dev)
    c.k = k_spec
    c.v = v_spec
    return c


def make_cache(idx, sgn, scl, capacity: int, layout: int) -> tq_cache:
    c = tq_cache()
    c.idx = _ptr(idx)
    c.sgn = _ptr(sgn)
    c.scl = _ptr(scl)
    c.capacity = capacity
    c.layout = layout
    return c
