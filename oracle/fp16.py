"""fp16 rounding of the stored per-vector scales (oracle; test infrastructure only).

Reading: the two per-vector scales (the norm ||x|| and the residual norm ||r||)
are stored as IEEE binary16, rounded to nearest with ties to even, directly from
the exact value.  Values above the largest finite binary16 (65504) saturate to
65504 and raise an overflow flag; the pages do not fix a scale format.
"""
from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0


def fp16_round(x):
    """Return (value float64, bits uint16, overflow bool) for non-negative x."""
    x = np.asarray(x, dtype=np.float64)
    over = x > FP16_MAX
    h = np.where(over, FP16_MAX, x).astype(np.float16)  # numpy: RNE from float64
    return h.astype(np.float64), h.view(np.uint16), over
