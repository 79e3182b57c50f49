"""Device-memory plumbing around the libtq entry points.

A ``TQSession`` owns the device copies of Pi, S and the tq_prepare blob, builds
the ``tq_config`` struct, allocates packed caches and workspaces with torch,
and forwards to the C entry points.  It performs no part of the quantize or
decode computation itself.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def cache_words(layout: int, heads: int, capacity: int, d: int, bits_mse: int):
    """(idx words, sgn words, scl halves) of one packed cache."""
    if layout == B.TQ_LAYOUT_TOKEN_MAJOR:
        return heads * capacity * bits_mse * (d // 32), heads * capacity * (d // 32), heads * capacity * 2
    return heads * (capacity // 32) * bits_mse * d, heads * (capacity // 32) * d, heads * capacity * 2


class PackedCache:
    """One packed cache (keys or values) in device memory, plus its C descriptor."""

    def __init__(self, heads, capacity, d, bits_mse, sketch, layout, device):
        if capacity % 32:
            raise ValueError("capacity must be a multiple of 32")
        ni, ns, nc = cache_words(layout, heads, capacity, d, bits_mse)
        self.idx = torch.zeros(ni, dtype=torch.int32, device=device)
        self.sgn = torch.zeros(ns if sketch else 4, dtype=torch.int32, device=device)
        self.scl = torch.zeros(nc, dtype=torch.int16, device=device)
        self.heads, self.capacity, self.d, self.bits_mse, self.sketch, self.layout = \
            heads, capacity, d, bits_mse, sketch, layout
        self.desc = B.make_cache(self.idx, self.sgn if sketch else None, self.scl, capacity, layout)

    def host_arrays(self):
        """Copy to host as numpy arrays shaped per layout (for checking)."""
        d, bq, cap, H = self.d, self.bits_mse, self.capacity, self.heads
        idx = self.idx.cpu().numpy().view(np.uint32)
        sgn = self.sgn.cpu().numpy().view(np.uint32) if self.sketch else None
        scl = self.scl.cpu().numpy().view(np.uint16).reshape(H, cap, 2)
        if self.layout == B.TQ_LAYOUT_TOKEN_MAJOR:
            idx = idx.reshape(H, cap, bq, d // 32)
            sgn = sgn.reshape(H, cap, d // 32) if sgn is not None else None
        else:
            idx = idx.reshape(H, cap // 32, bq, d)
            sgn = sgn.reshape(H, cap // 32, d) if sgn is not None else None
        return idx, sgn, scl

    def nbytes(self):
        return (self.idx.numel() * 4 + (self.sgn.numel() * 4 if self.sketch else 0)
                + self.scl.numel() * 2)


class TQSession:
    def __init__(self, d, n_kv_heads, n_q_heads, rot: np.ndarray, proj: np.ndarray,
                 k_bits=2, v_bits=2, k_sketch=1, v_sketch=1, law="gaussian", device="cuda"):
        self.d, self.n_kv_heads, self.n_q_heads, self.device = d, n_kv_heads, n_q_heads, device
        rot = np.ascontiguousarray(rot, dtype=np.float32)
        proj = np.ascontiguousarray(proj, dtype=np.float32)
        blob = np.zeros(B.tq_prepare_bytes(d, d), dtype=np.uint8)
        B.tq_prepare(rot, proj, d, d, blob)
        self.rot = torch.from_numpy(rot).to(device)
        self.proj = torch.from_numpy(proj).to(device)
        self.prep = torch.from_numpy(blob).to(device)
        self.k_spec = B.make_spec(k_bits, d, k_sketch, law)
        self.v_spec = B.make_spec(v_bits, d, v_sketch, law)
        self.cfg = B.make_config(d, n_kv_heads, n_q_heads, self.rot, self.proj, self.prep,
                                 self.k_spec, self.v_spec)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def new_caches(self, capacity):
        kc = PackedCache(self.n_kv_heads, capacity, self.d, self.k_spec.bits_mse, self.k_spec.sketch,
                         B.TQ_LAYOUT_TOKEN_MAJOR, self.device)
        vc = PackedCache(self.n_kv_heads, capacity, self.d, self.v_spec.bits_mse, self.v_spec.sketch,
                         B.TQ_LAYOUT_BLOCK32, self.device)
        return kc, vc

    @staticmethod
    def dtype_code(t: torch.Tensor) -> int:
        if t.dtype == torch.bfloat16:
            return B.TQ_BF16
        if t.dtype == torch.float32:
            return B.TQ_F32
        raise TypeError(f"unsupported input dtype {t.dtype}")

    def quantize(self, k, v, dst_token, kc: PackedCache, vc: PackedCache, dbg=None, stream=None):
        x = k if k is not None else v
        batch, heads, n_new, d = x.shape
        assert heads == self.n_kv_heads and d == self.d
        for t in (k, v):
            if t is not None:
                assert t.is_contiguous() and t.shape == x.shape and t.dtype == x.dtype
        assert dst_token.dtype == torch.int64 and dst_token.numel() == batch
        B.tq_quantize_kv(self.cfg, k, v, self.dtype_code(x), batch, n_new, dst_token,
                         kc.desc if kc is not None else None, vc.desc if vc is not None else None,
                         self.status, dbg, stream)

    def workspace(self, batch, max_len):
        n = B.tq_decode_workspace_bytes(self.cfg, batch, max_len)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def decode(self, q, seq_start, seq_len, max_len, kc: PackedCache, vc: PackedCache, out=None,
               workspace=None, sm_scale=0.0, stream=None, sparse_v=0.0):
        """Decode attention; sparse_v = tau > 0 runs Sparse V decode (values of
        positions whose weight relative to the largest is below tau left out)."""
        batch, hq, d = q.shape
        assert hq == self.n_q_heads and d == self.d and q.is_contiguous()
        assert seq_start.dtype == torch.int64 and seq_len.dtype == torch.int32
        if out is None:
            out = torch.empty(batch, hq, d, dtype=torch.float32, device=self.device)
        if workspace is None:
            workspace = self.workspace(batch, max_len)
        if sparse_v > 0.0:
            B.tq_decode_attention_sparse_v(self.cfg, q, self.dtype_code(q), batch, seq_start, seq_len, max_len,
                                           kc.desc, vc.desc, sm_scale, sparse_v, out, self.status, workspace,
                                           workspace.numel(), stream)
        else:
            B.tq_decode_attention(self.cfg, q, self.dtype_code(q), batch, seq_start, seq_len, max_len,
                                  kc.desc, vc.desc, sm_scale, out, self.status, workspace,
                                  workspace.numel(), stream)
        return out

    def score_workspace(self, n_q, max_n):
        n = B.tq_score_workspace_bytes(self.cfg, n_q, max_n)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def score_keys(self, q, kc: PackedCache, kv_head: int, start: int, n: int, out=None, workspace=None,
                   stream=None):
        """Inner products of q [n_q][d] (n_q a multiple of 8) with the packed keys in
        slots [start, start + n) of kv head kv_head: fp32 [n_q][n]."""
        n_q, d = q.shape
        assert d == self.d and q.is_contiguous()
        if out is None:
            out = torch.empty(n_q, n, dtype=torch.float32, device=self.device)
        if workspace is None:
            workspace = self.score_workspace(n_q, n)
        B.tq_score_keys(self.cfg, q, self.dtype_code(q), n_q, kc.desc, kv_head, start, n, out, self.status,
                        workspace, workspace.numel(), stream)
        return out
