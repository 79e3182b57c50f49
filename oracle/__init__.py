"""CPU oracle for online KV-cache compression and decode attention over it.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
bench's CPU-baseline leg use it.  It shares no code with the HIP library
(``kv_cache_online_amd``) and never imports it.

It is a plain, slow, float64 restatement of the method as the pages describe it.
Sources, cited by page title and section:

* [softpro §1.2] ast-softpro.ru, "Технология TurboQuant и её применение с
  локальными LLM", section 1.2 "Как работает TurboQuant": stage 1 (random
  orthogonal rotation, then a per-coordinate MSE-optimal Lloyd-Max scalar
  quantizer with b-1 bits) and stage 2 (residual r = x - DEQUANT_mse(Q_mse(x)),
  projection by a random Gaussian matrix S, only sign(S r) kept, and ||r||_2
  kept for reconstruction).
* [kiosk "Как работает"] kiosknews.app, "3 бита вместо 16: разбираем TurboQuant
  и когда его реально стоит включать", section "Как работает TurboQuant":
  rotation makes coordinates near-independent and near-normal; the Lloyd-Max
  codebook for that known distribution is computed once and stored; distortion
  within about 2.7x of the information-theoretic minimum.
* [kiosk "Python + HuggingFace"] same page, section "Python + HuggingFace": the
  community API returns (indices, norms) from quantize.

Readings taken where the pages are silent (each restated at its function):
the codebook is built for N(0, 1/d) applied to the unit-normalised rotated
vector; the per-vector norm ||x|| is stored as fp16 and the decision uses the
unrounded norm; midpoint ties go to the upper cell; the residual is taken in
the original space with the stored fp16 norm; S is m x d with N(0,1) entries
and m = d; sign(0) counts as +; the residual is reconstructed as
sqrt(pi/2)/m * ||r|| * S^T sign(S r) (the scaling that makes the inner-product
estimate unbiased); attention is softmax(q k^T / sqrt(d)) V with query head h
reading kv head h // G; a search score is <q, x_hat>.

Parity status: every function here is pinned by tests in ``tests/test_oracle_*``
against closed forms, brute force, numerical integration or library routines.
"""
from .codebook import build_codebook, build_codebook_sphere
from .fp16 import fp16_round
from .quantize import quantize, quantize_conditional
from .layout import (pack_token_major, unpack_token_major, pack_block32,
                     unpack_block32, record_bytes)
from .dequant import dequantize
from .attention import attention, attention_sparse_v
from .search import score_keys

__all__ = ["build_codebook", "build_codebook_sphere", "fp16_round", "quantize", "quantize_conditional",
           "pack_token_major", "unpack_token_major", "pack_block32", "unpack_block32",
           "record_bytes", "dequantize", "attention", "attention_sparse_v", "score_keys"]
