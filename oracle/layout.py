"""Bit-packed cache layouts (oracle; test infrastructure only).

A packed vector is b' index bit-planes over d coordinates, one sign plane over
m sketch rows (when the sign sketch is on), and two fp16 scales (||x||, ||r||).
That is b' + 1 bits per value plus 32 bits per vector: 3.25 bits per value for
d = 128, b = 3, i.e. 4.92x smaller than fp16, and 4.25 bits for b = 4 (3.76x).
These agree with the 5x and 3.8x quoted for the turbo3 / turbo4 formats on
kiosknews.app, "3 бита вместо 16: разбираем TurboQuant…", section "Что работает
прямо сейчас и как попробовать" / "llama.cpp".

Bit order (both layouts): bit k of a 32-bit word is its k-th least significant
bit.  Index plane q holds bit q of the cell index.  A sign bit is 1 when the
sketch coordinate is >= 0.

token-major (used for keys)  -- a token's planes are contiguous:
    idx[token, q, w]   bit k = plane q of coordinate 32*w + k
    sgn[token, w]      bit k = sign of sketch row 32*w + k
    scl[token, 2]      fp16 bits of (||x||, ||r||)
block32 (used for values)    -- 32 consecutive token slots share a word:
    idx[token // 32, q, j]   bit (token % 32) = plane q of coordinate j
    sgn[token // 32, i]      bit (token % 32) = sign of sketch row i
    scl[token, 2]            as above
"""
from __future__ import annotations

import numpy as np


def record_bytes(d: int, m: int, bits_mse: int, sketch: int = 1) -> int:
    """Bytes one packed vector occupies: index planes + sign plane + two fp16 scales."""
    return bits_mse * d // 8 + (m // 8 if sketch else 0) + 4


def _words_from_bits(bits):
    """bits[..., 32] (0/1) -> uint32 words, bit k = bits[..., k]."""
    b = np.asarray(bits, dtype=np.uint64)
    w = np.zeros(b.shape[:-1], dtype=np.uint64)
    for k in range(32):
        w |= b[..., k] << np.uint64(k)
    return w.astype(np.uint32)


def _bits_from_words(words):
    """uint32 words[...] -> bits[..., 32]."""
    w = np.asarray(words, dtype=np.uint32)
    return np.stack([(w >> np.uint32(k)) & np.uint32(1) for k in range(32)], axis=-1).astype(np.uint8)


def _scales(nu_bits, rho_bits):
    n = len(nu_bits)
    scl = np.zeros((n, 2), dtype=np.uint16)
    scl[:, 0] = nu_bits
    if rho_bits is not None:
        scl[:, 1] = rho_bits
    return scl


def pack_token_major(idx, sgn, nu_bits, rho_bits, bits_mse):
    """Codes idx[N, d], signs sgn[N, m] (or None) -> (idx_words, sgn_words, scl)."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    planes = np.stack([(idx >> q) & 1 for q in range(bits_mse)], axis=1)   # [N, b', d]
    iw = _words_from_bits(planes.reshape(n, bits_mse, d // 32, 32))
    sw = None
    if sgn is not None:
        s = np.asarray(sgn, dtype=np.uint8)
        sw = _words_from_bits(s.reshape(n, s.shape[1] // 32, 32))
    return iw, sw, _scales(nu_bits, rho_bits)


def unpack_token_major(idx_words, sgn_words, scl, bits_mse):
    """Inverse of pack_token_major -> (idx[N, d], sgn[N, m] bool or None, nu_bits, rho_bits)."""
    iw = np.asarray(idx_words, dtype=np.uint32)
    n = iw.shape[0]
    bits = _bits_from_words(iw).reshape(n, bits_mse, -1).astype(np.int64)   # [N, b', d]
    idx = np.zeros((n, bits.shape[2]), dtype=np.int64)
    for q in range(bits_mse):
        idx |= bits[:, q, :] << q
    sgn = None
    if sgn_words is not None:
        sgn = _bits_from_words(np.asarray(sgn_words, dtype=np.uint32)).reshape(n, -1).astype(bool)
    scl = np.asarray(scl, dtype=np.uint16)
    return idx, sgn, scl[:, 0].copy(), scl[:, 1].copy()


def pack_block32(idx, sgn, nu_bits, rho_bits, bits_mse):
    """Codes of N tokens (N a multiple of 32, token i in slot i) -> block32 arrays."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    if n % 32:
        raise ValueError("block32 packing needs a multiple of 32 tokens")
    nb = n // 32
    planes = np.stack([(idx >> q) & 1 for q in range(bits_mse)], axis=1)   # [N, b', d]
    planes = planes.reshape(nb, 32, bits_mse, d).transpose(0, 2, 3, 1)       # [nb, b', d, 32]
    iw = _words_from_bits(planes)
    sw = None
    if sgn is not None:
        s = np.asarray(sgn, dtype=np.uint8)
        s = s.reshape(nb, 32, s.shape[1]).transpose(0, 2, 1)                # [nb, m, 32]
        sw = _words_from_bits(s)
    return iw, sw, _scales(nu_bits, rho_bits)


def unpack_block32(idx_words, sgn_words, scl, bits_mse):
    """Inverse of pack_block32 -> (idx[N, d], sgn[N, m] or None, nu_bits, rho_bits)."""
    iw = np.asarray(idx_words, dtype=np.uint32)
    nb, bq, d = iw.shape
    bits = _bits_from_words(iw).astype(np.int64)            # [nb, b', d, 32]
    bits = bits.transpose(0, 3, 1, 2).reshape(nb * 32, bq, d)
    idx = np.zeros((nb * 32, d), dtype=np.int64)
    for q in range(bits_mse):
        idx |= bits[:, q, :] << q
    sgn = None
    if sgn_words is not None:
        sb = _bits_from_words(np.asarray(sgn_words, dtype=np.uint32))     # [nb, m, 32]
        sgn = sb.transpose(0, 2, 1).reshape(nb * 32, -1).astype(bool)
    scl = np.asarray(scl, dtype=np.uint16)
    return idx, sgn, scl[:, 0].copy(), scl[:, 1].copy()
