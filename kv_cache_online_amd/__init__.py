"""MI355X-native online KV-cache compression: quantize KV vectors into a
bit-packed cache and run decode attention over it (HIP kernels in libtq.so).

Importing the package loads libtq.so and fails loudly if it is not built.
"""
from . import binding
from .binding import (tq_build_codebook, tq_build_codebook_sphere, tq_prepare_bytes, tq_prepare,
                      tq_quantize_kv, tq_decode_workspace_bytes, tq_decode_attention, tq_score_workspace_bytes,
                      tq_score_keys, tq_status_string, TQError)

__all__ = ["binding", "tq_build_codebook", "tq_build_codebook_sphere", "tq_prepare_bytes", "tq_prepare",
           "tq_quantize_kv", "tq_decode_workspace_bytes", "tq_decode_attention",
           "tq_score_workspace_bytes", "tq_score_keys", "tq_status_string", "TQError"]
