"""Device-vs-oracle comparison protocol (test helper; uses the oracle).

Quantize (per vector set):
  1. cell indices: every mismatch must be a near-tie, |u - t_k| < 1e-4 sigma
     for the threshold t_k between the two cells (sigma = 1/sqrt(d)), and
     mismatches may cover at most 0.01% of index entries;
  2. ||x||: device fp32 value within 1e-5 relative; fp16 bits equal unless the
     exact value lies within 1e-5 relative of an fp16 rounding midpoint;
  3. vectors whose cells or stored norm differ are re-run through stage 2 with
     the device's choices imposed (one flipped cell changes the residual);
  4. signs against that (conditioned) oracle: mismatches must satisfy
     |(S r)_i| < 1e-4 ||r|| and cover at most 0.01% of sign entries;
  5. ||r||: within 1e-5 relative of the conditioned oracle; fp16 bits as in 2.
Every mismatch is listed in the report.
"""
from __future__ import annotations

import math

import numpy as np

import oracle as O

BAND = 1e-4
MAX_FRAC = 1e-4
REL = 1e-5


def _fp16_near_midpoint(v):
    lo, _, _ = O.fp16_round(v * (1 - REL))
    hi, _, _ = O.fp16_round(v * (1 + REL))
    return lo != hi


def quantize_parity(x64, rot, proj, cb, g_idx, g_sgn, g_nu_bits, g_rho_bits, g_dbg, sketch=True,
                    label=""):
    """Compare device outputs for vectors x64[N, d] against the oracle; return a report dict."""
    n, d = x64.shape
    sigma = 1 / math.sqrt(d)
    o = O.quantize(x64, rot, proj, cb, sketch=sketch)
    rep = {"label": label, "n_vectors": n, "errors": [], "index_mismatch": [], "sign_mismatch": [],
           "scale_near_ties": []}
    t = np.asarray(cb["boundaries"])
    # entries inside the near-tie band (for the record; only mismatches are listed)
    rep["index_entries"] = int(o["u"].size)
    near = np.zeros(o["u"].shape, dtype=bool)
    for tk in t:
        near |= np.abs(o["u"] - tk) < BAND * sigma
    rep["index_near_ties"] = int(near.sum())
    # 1. cell indices
    mm = np.argwhere(g_idx != o["idx"])
    for vi, j in mm:
        a, b = int(g_idx[vi, j]), int(o["idx"][vi, j])
        if abs(a - b) != 1:
            rep["errors"].append(f"index {vi},{j}: device {a} oracle {b} not adjacent")
            continue
        dist = abs(o["u"][vi, j] - t[min(a, b)]) / sigma
        rep["index_mismatch"].append((int(vi), int(j), b, a, float(dist)))
        if dist >= BAND:
            rep["errors"].append(f"index {vi},{j}: mismatch {dist:.3g} sigma from the threshold")
    frac_i = len(mm) / max(1, g_idx.size)
    rep["index_mismatch_frac"] = frac_i
    if frac_i > MAX_FRAC:
        rep["errors"].append(f"index mismatch fraction {frac_i:.3g} > {MAX_FRAC}")
    # 2. norms
    nu = o["nu"]
    gnu = g_dbg[:, 0].astype(np.float64)
    rel = np.abs(gnu - nu) / np.where(nu > 0, nu, 1)
    bad = np.argwhere(rel > REL).ravel()
    for vi in bad[:20]:
        rep["errors"].append(f"||x|| {vi}: device {gnu[vi]} oracle {nu[vi]} rel {rel[vi]:.3g}")
    rep["nu_max_rel"] = float(rel.max()) if n else 0.0
    nu_mm = np.argwhere(g_nu_bits != o["nu_bits"]).ravel()
    for vi in nu_mm:
        if _fp16_near_midpoint(nu[vi]):
            rep["scale_near_ties"].append(("nu", int(vi)))
        else:
            rep["errors"].append(f"fp16 ||x|| bits {vi}: device {g_nu_bits[vi]:#x} oracle {o['nu_bits'][vi]:#x}")
    if not sketch:
        rep["ok"] = not rep["errors"]
        return rep
    # 3. conditioning on the device's stage-1 choices
    cond = np.unique(np.concatenate([mm[:, 0], nu_mm])).astype(np.int64)
    p, rho, rho_bits, sgn = o["p"].copy(), o["rho"].copy(), o["rho_bits"].copy(), o["sgn"].copy()
    if len(cond):
        g_nu16 = np.asarray(g_nu_bits[cond], np.uint16).view(np.float16).astype(np.float64)
        c = O.quantize_conditional(x64[cond], rot, proj, cb, g_idx[cond], g_nu16)
        p[cond], rho[cond], rho_bits[cond], sgn[cond] = c["p"], c["rho"], c["rho_bits"], c["sgn"]
    rep["conditioned_vectors"] = int(len(cond))
    # 4. signs
    rep["sign_entries"] = int(sgn.size)
    rep["sign_near_ties"] = int(np.sum(np.abs(p) < BAND * rho[:, None]))
    sm = np.argwhere(g_sgn != sgn)
    for vi, i in sm:
        dist = abs(p[vi, i]) / max(rho[vi], 1e-300)
        rep["sign_mismatch"].append((int(vi), int(i), bool(sgn[vi, i]), float(dist)))
        if dist >= BAND:
            rep["errors"].append(f"sign {vi},{i}: mismatch {dist:.3g} rho from zero")
    frac_s = len(sm) / max(1, g_sgn.size)
    rep["sign_mismatch_frac"] = frac_s
    if frac_s > MAX_FRAC:
        rep["errors"].append(f"sign mismatch fraction {frac_s:.3g} > {MAX_FRAC}")
    # 5. residual norms
    grho = g_dbg[:, 1].astype(np.float64)
    rel = np.abs(grho - rho) / np.where(rho > 0, rho, 1)
    for vi in np.argwhere(rel > REL).ravel()[:20]:
        rep["errors"].append(f"||r|| {vi}: device {grho[vi]} oracle {rho[vi]} rel {rel[vi]:.3g}")
    rep["rho_max_rel"] = float(rel.max()) if n else 0.0
    for vi in np.argwhere(g_rho_bits != rho_bits).ravel():
        if _fp16_near_midpoint(rho[vi]):
            rep["scale_near_ties"].append(("rho", int(vi)))
        else:
            rep["errors"].append(f"fp16 ||r|| bits {vi}: device {g_rho_bits[vi]:#x} oracle {rho_bits[vi]:#x}")
    rep["ok"] = not rep["errors"]
    return rep


def records(rep, meta, tensor):
    """Every mismatch of a quantize report as a JSON-ready dict.  meta[vi] =
    (sequence, kv head, token) of compared vector vi."""
    out = []
    for vi, j, want, got, dist in rep["index_mismatch"]:
        s, h, tok = (int(v) for v in meta[vi])
        out.append({"kind": "index", "tensor": tensor, "sequence": s, "head": h, "token": tok, "coordinate": j,
                    "oracle": want, "gpu": got, "distance_sigma": dist})
    for vi, i, want, dist in rep["sign_mismatch"]:
        s, h, tok = (int(v) for v in meta[vi])
        out.append({"kind": "sign", "tensor": tensor, "sequence": s, "head": h, "token": tok, "coordinate": i,
                    "oracle": int(want), "gpu": int(not want), "distance_rho": dist})
    for kind, vi in rep["scale_near_ties"]:
        s, h, tok = (int(v) for v in meta[vi])
        out.append({"kind": f"fp16 {kind}", "tensor": tensor, "sequence": s, "head": h, "token": tok})
    return out


def summary(rep):
    keys = ("label", "n_vectors", "index_entries", "index_near_ties", "index_mismatch_frac", "sign_entries",
            "sign_near_ties", "sign_mismatch_frac", "nu_max_rel", "rho_max_rel", "conditioned_vectors")
    s = {k: rep.get(k) for k in keys}
    s["n_index_mismatch"] = len(rep["index_mismatch"])
    s["n_sign_mismatch"] = len(rep["sign_mismatch"])
    s["n_scale_near_ties"] = len(rep["scale_near_ties"])
    s["errors"] = rep["errors"][:10]
    return s


# ------------------------------------------------------------- cache reads ---
def unpack_tokens(idx_words, sgn_words, scl, layout, head, slots, bits_mse):
    """Codes/signs/scale bits of the given slots of one head, from host copies of a cache.

    layout 0: token-major arrays [H][cap][b'][d/32], [H][cap][m/32];
    layout 1: block32 arrays [H][cap/32][b'][d], [H][cap/32][m].
    """
    slots = np.asarray(slots, dtype=np.int64)
    if layout == 0:
        i, s, nb, rb = O.unpack_token_major(idx_words[head, slots], None if sgn_words is None
                                            else sgn_words[head, slots], scl[head, slots], bits_mse)
        return i, s, nb, rb
    blocks = np.unique(slots // 32)
    i, s, _, _ = O.unpack_block32(idx_words[head, blocks], None if sgn_words is None
                                  else sgn_words[head, blocks], np.zeros((len(blocks) * 32, 2), np.uint16),
                                  bits_mse)
    pos = {b: k for k, b in enumerate(blocks)}
    rows = np.array([pos[b] * 32 + (sl % 32) for b, sl in zip(slots // 32, slots)], dtype=np.int64)
    sc = scl[head, slots]
    return i[rows], (None if s is None else s[rows]), sc[:, 0].copy(), sc[:, 1].copy()


def f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def decode_reference(q64, kcache, vcache, k_bits, v_bits, k_sketch, v_sketch, rot, proj, cb_k, cb_v,
                     start, length, kv_heads):
    """Oracle attention for one sequence over the device-written packed caches.

    q64: [G * len(kv_heads), d] queries of the query heads mapped to kv_heads (in order);
    kcache / vcache: (idx, sgn, scl) host arrays.  Returns [len(kv_heads) * G, d].
    """
    kh, vh = dequantize_caches(kcache, vcache, k_bits, v_bits, k_sketch, v_sketch, rot, proj, cb_k, cb_v,
                               start, length, kv_heads)
    return O.attention(q64, kh, vh)


def dequantize_caches(kcache, vcache, k_bits, v_bits, k_sketch, v_sketch, rot, proj, cb_k, cb_v,
                      start, length, kv_heads):
    """The oracle's reconstruction of the keys and values the device-written caches
    hold for slots start .. start + length of kv_heads: ([H, T, d], [H, T, d])."""
    slots = np.arange(start, start + length)
    kh, vh = [], []
    for h in kv_heads:
        i, s, nb, rb = unpack_tokens(*kcache, 0, h, slots, k_bits)
        kh.append(O.dequantize(i, s if k_sketch else None, f16(nb), f16(rb) if k_sketch else None,
                               rot, proj, cb_k))
        i, s, nb, rb = unpack_tokens(*vcache, 1, h, slots, v_bits)
        vh.append(O.dequantize(i, s if v_sketch else None, f16(nb), f16(rb) if v_sketch else None,
                               rot, proj, cb_v))
    return np.stack(kh), np.stack(vh)
