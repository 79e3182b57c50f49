"""Property tests of the oracle (hypothesis; CPU).

Invariants the method fixes for any input, checked on generated cases:
- both cache layouts round-trip every code, sign and scale bit;
- stage 1 depends on x only through the direction of Pi x ([softpro §1.2]: the
  cell of a coordinate of the unit vector), so a positive power-of-two scale of x
  leaves every cell unchanged and scales the norm exactly;
- the Lloyd-Max codebook of a symmetric law is odd, so -x takes the mirrored
  cells L-1-idx, the negated residual and the flipped signs;
- attention is a weighted average over tokens, so permuting the tokens of K
  and V together leaves it unchanged.
([softpro §1.2] = ast-softpro.ru, "Технология TurboQuant и её применение с
локальными LLM", section 1.2.)
"""
import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import workloads as W
from oracle import (attention, build_codebook, pack_block32, pack_token_major, quantize, unpack_block32,
                    unpack_token_major)

SETTINGS = settings(max_examples=25, deadline=None)


@SETTINGS
@given(d=st.sampled_from([64, 128, 256]), blocks=st.integers(1, 3), bits=st.integers(1, 3),
       sketch=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_layouts_round_trip(d, blocks, bits, sketch, seed):
    rng = np.random.default_rng(seed)
    n = 32 * blocks
    idx = rng.integers(0, 1 << bits, size=(n, d))
    sgn = rng.integers(0, 2, size=(n, d)).astype(bool) if sketch else None
    nb = rng.integers(0, 1 << 16, size=n).astype(np.uint16)
    rb = rng.integers(0, 1 << 16, size=n).astype(np.uint16)
    for pack, unpack in ((pack_token_major, unpack_token_major), (pack_block32, unpack_block32)):
        i2, s2, n2, r2 = unpack(*pack(idx, sgn, nb, rb, bits), bits)
        np.testing.assert_array_equal(np.asarray(i2), idx)
        if sketch:
            np.testing.assert_array_equal(np.asarray(s2).astype(bool), sgn)
        np.testing.assert_array_equal(np.asarray(n2, dtype=np.uint16), nb)
        np.testing.assert_array_equal(np.asarray(r2, dtype=np.uint16), rb)


def _setup(d, bits, seed):
    P = W.rotation(d, 100 + d)
    S = W.sketch(d, d, 100 + d)
    cb = build_codebook(bits, 1 / math.sqrt(d))
    x = np.random.default_rng(seed).standard_normal((6, d)) * np.exp(np.random.default_rng(seed + 1).uniform(-2, 2, d))
    return P, S, cb, x


@SETTINGS
@given(d=st.sampled_from([64, 128]), bits=st.integers(1, 3), k=st.integers(-30, 30), seed=st.integers(0, 10**6))
def test_stage1_invariant_to_positive_scale(d, bits, k, seed):
    P, S, cb, x = _setup(d, bits, seed)
    a, b = quantize(x, P, S, cb), quantize(x * 2.0 ** k, P, S, cb)
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(b["nu"], a["nu"] * 2.0 ** k)   # exact: a power-of-two scale


@SETTINGS
@given(d=st.sampled_from([64, 128]), bits=st.integers(1, 3), seed=st.integers(0, 10**6))
def test_negation_mirrors_cells_and_flips_signs(d, bits, seed):
    P, S, cb, x = _setup(d, bits, seed)
    a, b = quantize(x, P, S, cb), quantize(-x, P, S, cb)
    L = cb["levels"]
    np.testing.assert_array_equal(b["idx"], L - 1 - a["idx"])   # no coordinate sits exactly on a midpoint
    np.testing.assert_array_equal(b["nu"], a["nu"])
    np.testing.assert_array_equal(b["rho"], a["rho"])
    nz = a["p"] != 0
    np.testing.assert_array_equal(b["sgn"][nz], ~a["sgn"][nz])


@SETTINGS
@given(t=st.integers(1, 40), g=st.sampled_from([1, 2, 4]), seed=st.integers(0, 10**6))
def test_attention_invariant_to_token_order(t, g, seed):
    rng = np.random.default_rng(seed)
    d, hkv = 16, 2
    q = rng.standard_normal((hkv * g, d))
    k = rng.standard_normal((hkv, t, d)) * 2
    v = rng.standard_normal((hkv, t, d))
    perm = rng.permutation(t)
    np.testing.assert_allclose(attention(q, k[:, perm], v[:, perm]), attention(q, k, v), rtol=1e-12, atol=1e-13)
