"""Seeded synthetic inputs for the KV-cache compression hot path.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
bench.  It holds no arithmetic of the compression method itself: it only draws
random numbers, scales them, and rounds them to the storage dtype.  The random
matrices that the method needs (the rotation and the Gaussian sketch) are drawn
here and handed to both sides as inputs.

Workloads stand in for the model shapes the pages quote (Llama-3.1-8B / 70B
style attention layers); no dataset or weights are used.

Random streams: every draw comes from ``numpy.random.default_rng`` seeded with
``[workload_id, stream, *sub]``.  Streams: 0 rotation, 1 sketch, 2 keys,
3 values, 4 queries, 5 channel scales, 6 outlier channels, 7 sequence lengths,
8 appended (incremental) keys/values.  Keys and values are drawn per
(sequence, kv-head) so that any chunk can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

STREAM_ROT, STREAM_SKETCH, STREAM_K, STREAM_V, STREAM_Q = 0, 1, 2, 3, 4
STREAM_SCALE, STREAM_OUTLIER, STREAM_LENS, STREAM_NEW = 5, 6, 7, 8


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int                 # workload id (seed root)
    name: str
    batch: int               # sequences
    n_kv_heads: int
    n_q_heads: int
    seq_len: int             # tokens per sequence (max for ragged)
    d: int                   # head dim
    bits_mse: int            # b' index bits per coordinate
    sketch: int = 1          # 1: 1-bit sign sketch stored; total bits b = b' + 1
    dtype: str = "bf16"      # storage dtype of K, V, Q inputs: "bf16" | "f32"
    scaled: bool = True      # per-channel log-uniform scales in [0.5, 4]
    outliers: int = 0        # outlier channels per (tensor, head)
    outlier_mult: float = 20.0
    ragged: bool = False     # lengths uniform in [min_len, seq_len]
    min_len: int = 0
    incremental: int = 0     # tokens appended per sequence (after prefill)

    @property
    def bits(self) -> int:
        return self.bits_mse + self.sketch

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def m(self) -> int:
        return self.d


# The five workloads of the hot-path scope (shapes, dtypes, value models).
WORKLOADS = {
    1: Workload(1, "single-head-d128-1k-f32", batch=1, n_kv_heads=1, n_q_heads=4,
                seq_len=1024, d=128, bits_mse=2, dtype="f32", scaled=False),
    2: Workload(2, "llama8b-layer-32k-b4", batch=1, n_kv_heads=8, n_q_heads=32,
                seq_len=32768, d=128, bits_mse=3, outliers=2),
    3: Workload(3, "llama70b-layer-128k-x4-b3", batch=4, n_kv_heads=8, n_q_heads=64,
                seq_len=131072, d=128, bits_mse=2, outliers=2),
    4: Workload(4, "ragged-64seq-1k-16k-b3", batch=64, n_kv_heads=8, n_q_heads=32,
                seq_len=16384, d=128, bits_mse=2, ragged=True, min_len=1024,
                incremental=1),
    5: Workload(5, "wide-d256-64k-x2-b2", batch=2, n_kv_heads=4, n_q_heads=16,
                seq_len=65536, d=256, bits_mse=1, scaled=False, outliers=4),
}


def rng(wid: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([wid, stream, *sub])


# ---------------------------------------------------------------- rounding ---
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------ random matrices ---
def rotation(d: int, wid: int) -> np.ndarray:
    """Random orthogonal d x d matrix, stored as float32.

    Q from the QR factorisation of a seeded N(0,1) matrix, with column signs
    fixed so that diag(R) > 0 (the Haar-distributed choice); the rotation is
    applied as z = Pi @ x.
    """
    g = rng(wid, STREAM_ROT).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return q.astype(np.float32)


def sketch(m: int, d: int, wid: int) -> np.ndarray:
    """Seeded Gaussian m x d matrix with N(0,1) entries, stored as float32."""
    return rng(wid, STREAM_SKETCH).standard_normal((m, d)).astype(np.float32)


# --------------------------------------------------------- value models ---
def channel_scales(w: Workload, tensor: int, head: int) -> np.ndarray:
    """Per-channel standard deviations of one (tensor, kv-head); tensor 0=K, 1=V."""
    d = w.d
    if w.scaled:
        s = np.exp(rng(w.wid, STREAM_SCALE, tensor, head).uniform(math.log(0.5), math.log(4.0), d))
    else:
        s = np.ones(d)
    if w.outliers:
        ch = rng(w.wid, STREAM_OUTLIER, tensor, head).choice(d, size=w.outliers, replace=False)
        s = s.copy()
        s[ch] *= w.outlier_mult
    return s


def _round_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 draw -> fp32 -> storage dtype.  bf16 is returned as uint16 bits."""
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    return f32_to_bf16_bits(x32)


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs."""
    if dtype == "f32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    return bf16_bits_to_f32(stored).astype(np.float64)


def kv_chunk(w: Workload, tensor: int, seq: int, head: int, n_tokens: Optional[int] = None,
             stream: Optional[int] = None) -> np.ndarray:
    """Stored K (tensor=0) or V (tensor=1) vectors of one (sequence, kv-head).

    Returns [n_tokens, d] in the storage dtype (uint16 bf16 bits or float32).
    Values: N(0, s_c^2) per channel c.
    """
    n = w.seq_len if n_tokens is None else n_tokens
    st = (STREAM_K if tensor == 0 else STREAM_V) if stream is None else stream
    g = rng(w.wid, st, seq, head, tensor).standard_normal((n, w.d))
    g *= channel_scales(w, tensor, head)[None, :]
    return _round_storage(g, w.dtype)


def new_tokens(w: Workload, tensor: int, seq: int, head: int) -> np.ndarray:
    """Appended K/V tokens of one (sequence, kv-head) for incremental quantize."""
    return kv_chunk(w, tensor, seq, head, n_tokens=max(w.incremental, 1), stream=STREAM_NEW)


def queries(w: Workload) -> np.ndarray:
    """One decode query per (sequence, query head): [batch, n_q_heads, d], N(0,1)."""
    g = rng(w.wid, STREAM_Q).standard_normal((w.batch, w.n_q_heads, w.d))
    return _round_storage(g, w.dtype)


def seq_lengths(w: Workload) -> np.ndarray:
    """Cached tokens per sequence before any append: int64 [batch]."""
    if not w.ragged:
        return np.full(w.batch, w.seq_len, dtype=np.int64)
    return rng(w.wid, STREAM_LENS).integers(w.min_len, w.seq_len, size=w.batch,
                                            endpoint=True).astype(np.int64)


def seq_starts(lens: np.ndarray, align: int = 64) -> np.ndarray:
    """Start slots of the sequences on one flat token axis, each padded to `align`."""
    cap = (np.asarray(lens, dtype=np.int64) + align) // align * align  # room for one append
    return np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)


def capacity(lens: np.ndarray, align: int = 64) -> int:
    cap = (np.asarray(lens, dtype=np.int64) + align) // align * align
    return int(cap.sum())


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same value model and bits) for fast tests."""
    return dataclasses.replace(w, **kw)


def kv_batch(w: Workload, tensor: int, n_tokens: Optional[int] = None, batch: Optional[int] = None,
             threads: int = 8) -> np.ndarray:
    """Stored K or V of the whole batch: [batch][n_kv_heads][n_tokens][d] (storage dtype).

    Chunks are independent streams, drawn in parallel threads.
    """
    import concurrent.futures as cf
    nb = w.batch if batch is None else batch
    n = w.seq_len if n_tokens is None else n_tokens
    dt = np.float32 if w.dtype == "f32" else np.uint16
    out = np.empty((nb, w.n_kv_heads, n, w.d), dtype=dt)

    def one(job):
        s, h = job
        out[s, h] = kv_chunk(w, tensor, s, h, n_tokens=n)

    jobs = [(s, h) for s in range(nb) for h in range(w.n_kv_heads)]
    with cf.ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, jobs))
    return out
