#!/usr/bin/env python3
"""Bench of the online KV-cache compression hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input: the
step's new key and value vectors are quantized into the packed caches
(tq_quantize_kv) and one decode-attention step (one query per query head)
reads the packed caches (tq_decode_attention).

Default workload: Llama-3.1-70B-shaped attention layer, decode batch 4, 128K
context per sequence, 8 kv heads, 64 query heads (GQA 8), d = 128, bf16 K/V,
b = 3 (2 index bits + 1 sign bit).  The 131,071 earlier tokens of every
sequence are quantized as untimed setup; a step quantizes each sequence's
newest token (K and V of every kv head) into its slot and decodes over all
131,072 tokens: 436.2 MB of packed cache per decode.

--workload 4: 64 ragged sequences of 1K-16K tokens (GQA 4, b = 3): a step
quantizes one appended token per sequence and decodes over len + 1.
--workload 1, 2, 5: full-context workloads, where a step quantizes the whole
context (K and V of every kv head) and then decodes once.

Inputs and caches rotate through enough copies (>= 1 GiB) that the cache a
decode reads is not still in the 256 MB last-level cache.

Prints one JSON line.  value = packed-KV decode-attention GB/s (algorithmic
packed bytes read per decode / decode call time); the quantize rate (token
positions per second, each position = K and V of every kv head) is reported
beside it.  Kernel durations come from HIP events on the launch stream, created
without the system-scope fence a default event adds (timing only).

Other modes: --search (inner-product search over a 2^23-key packed index,
tq_score_keys); --calibrate-copy and --traffic (HBM counter calibration and
the traffic table, for the profiles).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, spec
BF16_MFMA_PEAK_TFLOPS = 2500.0 # MI355X dense bf16 matrix, spec
METRIC = "packed-KV decode-attention GB/s (% HBM peak); KV quantize tokens/s"
SEARCH_WORKLOAD = "search-d128-8m-b4"


# Sources each kernel family is built from (a counter entry stays valid while they are unchanged).
SHARED_SOURCES = ("tq_common.h", "tq_device.h", "tq_host.cpp")
FAMILY_SOURCES = {"decode": ("tq_decode_fast.hip",) + SHARED_SOURCES,
                  "quantize": ("tq_quantize_fast.hip",) + SHARED_SOURCES}


def source_hash(files=None):
    """sha256 (16 hex digits) of the library sources, or of the given csrc files."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_online_amd", "csrc")
    for f in sorted(files if files is not None else os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def kernel_family(name):
    return "quantize" if name.startswith("quantize") else "decode"


def family_hash(name):
    return source_hash(FAMILY_SOURCES[kernel_family(name)])


def packed_record_bytes(d, m, bits_mse, sketch):
    """Bytes of one packed vector in the cache layout: b' index planes of d bits,
    a sign plane of m bits when the sketch is kept, two fp16 scales."""
    return bits_mse * d // 8 + (m // 8 if sketch else 0) + 4


def traffic_for(prefixes, workload):
    """HBM bytes per call (sum over the call's kernels, each by name prefix) from
    the committed rocprofv3 counter runs, if they were taken on this workload and
    on the kernel family's current sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        t = json.load(open(p))
    except (OSError, ValueError):
        return None
    if workload not in t.get("workloads", {}):
        return None
    ks = t["workloads"][workload].get("kernels", {})
    total = 0.0
    for pre, n in prefixes:
        hit = [v for k, v in ks.items() if k.startswith(pre)]
        if not hit or hit[0].get("source_hash") != family_hash(pre):
            return None
        total += n * hit[0]["bytes"]
    return total


class HipEvent:
    """A timing event on a HIP stream, created with hipEventDisableSystemFence.

    A default event makes a system-scope release when it is recorded, which
    writes back and invalidates the caches between the kernels it separates and
    adds its own time to the interval it measures; an event made only for timing
    needs no such fence (the HIP runtime's own description of the flag).  Same
    interface as torch.cuda.Event(enable_timing=True): record(stream) and
    elapsed_time(end) in milliseconds."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            import torch
            torch.cuda.init()
            # the HIP runtime torch has loaded (resolved by its soname)
            lib = ctypes.CDLL("libamdhip64.so.7")
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            for f in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
                getattr(lib, f).restype = ctypes.c_int
            cls._hip = lib
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        rc = self._lib().hipEventCreateWithFlags(ctypes.byref(self._ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream()
        rc = self._lib().hipEventRecord(self._ev, st.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_time(self, end):
        import ctypes
        ms = ctypes.c_float()
        rc = self._lib().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and getattr(self, "_ev", None) is not None and self._ev.value:
            self._hip.hipEventDestroy(self._ev)


def copy_calibration(nbytes=1 << 30, reps=5):
    """Plain device-to-device copies of a known size, for scaling HBM byte counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, workload):
    """profiles/traffic.json from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of
    this bench and of copy_calibration (counters in KiB per dispatch).  Each
    counter is scaled by bytes / counter of the plain copy: FETCH against the
    bytes the copy reads, WRITE against the bytes it writes."""
    import csv
    import re

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") != counter:
                continue
            k = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].split("::")[-1]
            vals.setdefault(k, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sorted(v)[len(v) // 2] for k, v in vals.items()}

    cf = per_kernel(copy_fetch_csv, "FETCH_SIZE")
    cw = per_kernel(copy_write_csv, "WRITE_SIZE")
    ck = max(cf, key=cf.get)                      # the copy is the largest dispatch
    f_scale, w_scale = copy_bytes / cf[ck], copy_bytes / cw[ck]
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    kernels = {}
    for k in fetch:
        if k in write and k.startswith(("quantize", "decode")):
            kernels[k] = {"fetch_bytes": fetch[k] * f_scale, "write_bytes": write[k] * w_scale,
                          "bytes": fetch[k] * f_scale + write[k] * w_scale, "source_hash": family_hash(k)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    workloads = {}
    if os.path.exists(path):   # keep the other workloads' entries (each carries its own source hash)
        try:
            workloads = json.load(open(path)).get("workloads", {})
        except (OSError, ValueError):
            pass
    workloads[workload] = {"kernels": kernels}
    out = {"copy_kernel": ck, "copy_bytes": copy_bytes,
           "fetch_scale": f_scale, "write_scale": w_scale, "workloads": workloads}
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def quality_vs_unquantized(w, ctx, Qn, out):
    """The decode output against softmax attention over the unquantized K, V and q
    (float64 on the host, scale 1/sqrt(d)): relative L2 error and cosine per query
    head.  ctx(b, h) gives the stored K and V of that sequence's decode context.
    Reported, not pass/fail."""
    import workloads as W
    G = w.n_q_heads // w.n_kv_heads
    scale = 1.0 / math.sqrt(w.d)
    rel, cos = [], []
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            ks, vs = ctx(b, h)
            k, v = W.to_f64(ks, w.dtype), W.to_f64(vs, w.dtype)
            q = W.to_f64(Qn[b, h * G:(h + 1) * G], w.dtype)
            sc = (q @ k.T) * scale
            sc -= sc.max(axis=1, keepdims=True)
            pr = np.exp(sc)
            ref = (pr @ v) / pr.sum(axis=1, keepdims=True)
            got = out[b, h * G:(h + 1) * G].astype(np.float64)
            rel.extend(np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1))
            cos.extend(np.sum(got * ref, axis=1) / (np.linalg.norm(got, axis=1) * np.linalg.norm(ref, axis=1)))
    return {"reference": "softmax attention over the unquantized K, V, q (float64, host)",
            "query_heads": len(rel), "rel_l2_mean": float(np.mean(rel)), "rel_l2_max": float(np.max(rel)),
            "cosine_min": float(np.min(cos))}


def score_fidelity(w, sess, kc, Qn, ctx, starts, b=0):
    """The scores the decode works from against the exact ones, for sequence b:
    the device's inner products <q, k~> with the packed keys (tq_score_keys)
    against float64 q.k over the stored keys, both in logit units (divided by
    sqrt(d)), for every query head.  Reports the RMS logit error, the spread
    (standard deviation over tokens) of the exact logits, how often the largest
    logit stays on the same token, and the median gap between the two largest
    exact logits.  A softmax over many tokens turns a logit error comparable to
    that gap into a different mixture of values."""
    import torch
    import workloads as W
    G, d = w.n_q_heads // w.n_kv_heads, w.d
    err2, spread, same, gaps, n_e = 0.0, [], 0, [], 0
    for h in range(w.n_kv_heads):
        k = W.to_f64(ctx(b, h)[0], w.dtype)
        q_st = Qn[b, h * G:(h + 1) * G]
        qp = np.zeros(((G + 7) // 8 * 8, d), dtype=q_st.dtype)
        qp[:G] = q_st
        qd = torch.from_numpy(qp).to(sess.device)
        qd = qd.view(torch.bfloat16) if qp.dtype == np.uint16 else qd
        got = sess.score_keys(qd, kc, h, int(starts[b]), len(k)).cpu().numpy()[:G].astype(np.float64)
        ref = W.to_f64(q_st, w.dtype) @ k.T
        e = (got - ref) / math.sqrt(d)
        err2 += float(np.sum(e * e))
        n_e += e.size
        lg = ref / math.sqrt(d)
        spread.extend(lg.std(axis=1))
        same += int(np.sum(np.argmax(got, axis=1) == np.argmax(ref, axis=1)))
        top2 = np.sort(lg, axis=1)[:, -2:]
        gaps.extend(top2[:, 1] - top2[:, 0])
    return {"sequence": b, "tokens": int(len(k)), "query_heads": len(spread),
            "logit_err_rms": math.sqrt(err2 / n_e), "logit_std_mean": float(np.mean(spread)),
            "top1_same_frac": same / len(spread), "top2_gap_median": float(np.median(gaps))}


def quality_report(w, rot, proj, ctx, Qn, out, decode_mse_only, sess=None, kc=None, starts=None):
    """quality_vs_unquantized for the workload's preset and, beside it, for the
    same index bits with the residual sketch off (MSE-only; decode_mse_only(session)
    fills that session's caches the same way and returns its decode output and key
    cache): the sketch makes the inner products unbiased at the price of variance,
    which the softmax amplifies where the scores are spread (outlier channels).
    Given the preset's session, its key cache kc and the sequence starts, each
    entry also carries score_fidelity for sequence 0."""
    from kv_cache_online_amd.session import TQSession
    rep = {"preset": quality_vs_unquantized(w, ctx, Qn, out)}
    if sess is not None:
        rep["preset"]["scores"] = score_fidelity(w, sess, kc, Qn, ctx, starts)
    if w.sketch:
        s2 = TQSession(w.d, w.n_kv_heads, w.n_q_heads, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse,
                       k_sketch=0, v_sketch=0)
        out2, kc2 = decode_mse_only(s2)
        key = f"mse_only_{w.bits_mse}bit"
        rep[key] = quality_vs_unquantized(w, ctx, Qn, out2)
        if sess is not None:
            rep[key]["scores"] = score_fidelity(w, s2, kc2, Qn, ctx, starts)
    return rep


def oracle_threads():
    """Threads the oracle's NumPy/BLAS calls use (the BLAS pool, else the CPUs this process may run on)."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max([i.get("num_threads", 0) for i in blas] + [1])
    except Exception:
        pass
    return cores


def blas_vendor():
    """The BLAS library NumPy was built against (name and version)."""
    try:
        cfg = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{cfg.get('name', '?')} {cfg.get('version', '')}".strip()
    except Exception:
        return "unknown"


def copy_peak_gbs(nbytes=1 << 30, reps=5):
    """Measured HBM bandwidth of a plain device-to-device copy (bytes read + written
    per second, best of reps), the practical ceiling beside the 8 TB/s spec."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = HipEvent(), HipEvent()
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del a, b
    return 2 * nbytes / best / 1e9


def cpu_baseline(w, rot, proj, seconds):
    """Time the oracle (float64 NumPy) on a bounded sample of the same workload."""
    import oracle as O
    import workloads as W
    cores = oracle_threads()
    cb = O.build_codebook(w.bits_mse, 1 / math.sqrt(w.d))
    # decode: one kv head over the full context (oracle-packed cache), G query heads
    T = w.seq_len
    K = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=T), w.dtype)
    V = W.to_f64(W.kv_chunk(w, 1, 0, 0, n_tokens=T), w.dtype)
    qk = O.quantize(K, rot, proj, cb)
    qv = O.quantize(V, rot, proj, cb)
    kp = O.pack_token_major(qk["idx"], qk["sgn"], qk["nu_bits"], qk["rho_bits"], w.bits_mse)
    vp = O.pack_block32(qv["idx"], qv["sgn"], qv["nu_bits"], qv["rho_bits"], w.bits_mse)
    q = W.to_f64(W.queries(w)[0, :w.group], w.dtype)
    f16 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    reps, t_dec = 0, 0.0
    t_start = time.perf_counter()
    while reps < 1 or (time.perf_counter() - t_start < seconds / 2 and reps < 40):
        t0 = time.perf_counter()
        i, s, nb, rb = O.unpack_token_major(*kp, w.bits_mse)
        kh = O.dequantize(i, s, f16(nb), f16(rb), rot, proj, cb)
        i, s, nb, rb = O.unpack_block32(*vp, w.bits_mse)
        vh = O.dequantize(i, s, f16(nb), f16(rb), rot, proj, cb)
        O.attention(q, kh[None], vh[None])
        t_dec += time.perf_counter() - t0
        reps += 1
    rec = O.record_bytes(w.d, w.m, w.bits_mse, w.sketch)
    dec_gbs = reps * T * 2 * rec / t_dec / 1e9
    # quantize: token positions (K and V of every kv head) on a sample of vectors
    n_pos = 49152
    X = W.to_f64(W.kv_chunk(w, 0, 0, 1, n_tokens=n_pos * w.n_kv_heads * 2), w.dtype)
    t0 = time.perf_counter()
    qq = O.quantize(X, rot, proj, cb)
    O.pack_token_major(qq["idx"], qq["sgn"], qq["nu_bits"], qq["rho_bits"], w.bits_mse)
    tq = time.perf_counter() - t0
    return {"value": dec_gbs, "unit": "GB/s", "cores": cores, "kind": "oracle", "blas": blas_vendor(),
            "sample": (f"decode: unpack + float64 dequantize + attention over one kv head x {T} tokens "
                       f"(K and V), {w.group} query heads, {reps} reps, {t_dec:.1f} s; quantize: "
                       f"{n_pos} token positions ({n_pos * w.n_kv_heads * 2} vectors), {tq:.1f} s"),
            "quantize_tokens_per_s": n_pos / tq}


def search_cpu_baseline(w, rot, proj, Qn, n_q, seconds):
    """Time the oracle's search scores (unpack + float64 dequantize + q @ k^T) on a
    bounded sample of keys."""
    import oracle as O
    import workloads as W
    cores = oracle_threads()
    cb = O.build_codebook(w.bits_mse, 1 / math.sqrt(w.d))
    n = 65536
    K = W.to_f64(W.kv_chunk(w, 0, 0, 0, n_tokens=n), w.dtype)
    qk = O.quantize(K, rot, proj, cb)
    kp = O.pack_token_major(qk["idx"], qk["sgn"], qk["nu_bits"], qk["rho_bits"], w.bits_mse)
    q = W.to_f64(Qn[0, :n_q], w.dtype)
    f16 = lambda b: np.asarray(b, np.uint16).view(np.float16).astype(np.float64)
    reps, t = 0, 0.0
    while reps < 1 or (t < seconds and reps < 40):
        t0 = time.perf_counter()
        i, sg, nb, rb = O.unpack_token_major(*kp, w.bits_mse)
        O.score_keys(q, i, sg, f16(nb), f16(rb), rot, proj, cb)
        t += time.perf_counter() - t0
        reps += 1
    rec = O.record_bytes(w.d, w.m, w.bits_mse, w.sketch)
    return {"value": reps * n * (rec + 4 * n_q) / t / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "blas": blas_vendor(),
            "sample": f"{n} packed keys x {n_q} queries: unpack + float64 dequantize + scores, {reps} reps, "
                      f"{t:.1f} s"}


def bench_search(args):
    """Inner-product search over packed keys (tq_score_keys): a 2^23-vector key
    index (the keys of the default workload, repeated), scored by n_q queries per
    call for each n_q of --search-nq (default 8 and 32).  Algorithmic bytes per call: the packed keys read once plus
    the fp32 scores written."""
    import torch
    import workloads as W
    from kv_cache_online_amd.session import TQSession

    w = W.WORKLOADS[2]
    rot, proj = W.rotation(w.d, w.wid), W.sketch(w.m, w.d, w.wid)
    s = TQSession(w.d, 1, 8, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse, k_sketch=w.sketch,
                  v_sketch=w.sketch)
    Kn, Qn = W.kv_batch(w, 0), W.queries(w)
    base = w.n_kv_heads * w.seq_len                       # 2^18 key vectors
    N = 1 << 23
    K = torch.from_numpy(np.ascontiguousarray(Kn)).cuda().view(torch.bfloat16).reshape(1, 1, base, w.d)
    kc = s.new_caches(N)[0]
    for c in range(N // base):
        s.quantize(K, None, torch.tensor([c * base], dtype=torch.int64, device="cuda"), kc, None)
    del K
    stream = torch.cuda.current_stream()
    rec = packed_record_bytes(w.d, w.m, w.bits_mse, w.sketch)
    Q = torch.from_numpy(np.ascontiguousarray(Qn)).cuda().view(torch.bfloat16).reshape(-1, w.d)
    runs = []
    for n_q in args.search_nq:
        q = Q[:n_q].contiguous()
        out = torch.empty(n_q, N, dtype=torch.float32, device="cuda")
        ws = s.score_workspace(n_q, N)
        for _ in range(args.warmup):
            s.score_keys(q, kc, 0, 0, N, out=out, workspace=ws, stream=stream)
        torch.cuda.synchronize()
        ev = [[HipEvent() for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            ev[i][0].record(stream)
            s.score_keys(q, kc, 0, 0, N, out=out, workspace=ws, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        t = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e-3
        assert torch.isfinite(out).all(), "scores not finite"
        nbytes = N * rec + n_q * N * 4 + n_q * w.d * 2
        gbs = nbytes / t / 1e9
        runs.append({"n_q": n_q, "avg_call_s": t, "bytes_per_call": nbytes, "GBps": gbs,
                     "frac": gbs / HBM_PEAK_GBS, "scores_per_s": n_q * N / t,
                     "key_GBps": N * rec / t / 1e9})
        del out
    status = int(s.status.item()) & 0xFFFFFFFF
    assert status == 0, f"device status flags {status:#x}"
    top = runs[-1]
    res = {
        "metric": "packed-key inner-product search GB/s (packed keys read + fp32 scores written)",
        "value": top["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": top["avg_call_s"] * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16+i8", "data": "synthetic (keys of the default workload, repeated)",
        "config": {"workload": SEARCH_WORKLOAD, "n_keys": N, "head_dim": w.d, "bits": w.bits, "n_q": top["n_q"]},
        "roofline": {"bound": "hbm", "achieved": top["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": top["frac"],
                     "traffic": traffic_for([("decode_qprep", 1), ("decode_partial", 1)], SEARCH_WORKLOAD),
                     "kernel": "tq_score_keys call: query prep + split scoring", "bytes_per_launch": top["bytes_per_call"],
                     "avg_launch_s": top["avg_call_s"]},
        "runs": runs, "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = search_cpu_baseline(w, rot, proj, Qn, top["n_q"], args.cpu_seconds)
    print(json.dumps(res), flush=True)


def timed_steps(args, step):
    """W untimed warmup steps, then K timed steps; step(i, events) records three
    events on the launch stream (before the quantize call, between the calls, after
    the decode call).  Returns per-step quantize and decode call times (s) and the
    wall time per step."""
    import torch
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[HipEvent() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    qt = np.array([e[0].elapsed_time(e[1]) for e in events]) * 1e-3
    dt = np.array([e[1].elapsed_time(e[2]) for e in events]) * 1e-3
    return qt, dt, (t1 - t0) / args.steps


def roofline_decode(w, packed_bytes, d_avg):
    dec_gbs = packed_bytes / d_avg / 1e9
    return {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": dec_gbs / HBM_PEAK_GBS,
            "traffic": traffic_for([("decode_qprep", 1), ("decode_partial", 1), ("decode_merge", 1)], w.name),
            "kernel": "tq_decode_attention call (query prep, split pass, merge), timed as one launch",
            "bytes_per_launch": packed_bytes, "avg_launch_s": d_avg}


def bench_context(args, w, s, rot, proj):
    """Workloads 1, 2, 5: a step quantizes the whole context (K and V of every kv
    head: one tq_quantize_kv call, one launch of the quantize kernel for both) and
    then decodes once over a cache written several steps earlier."""
    import torch
    import workloads as W
    B, H, T, d = w.batch, w.n_kv_heads, w.seq_len, w.d
    lens = W.seq_lengths(w)
    cap = W.capacity(lens)
    starts = W.seq_starts(lens)
    esize = 4 if w.dtype == "f32" else 2
    rec = packed_record_bytes(d, w.m, w.bits_mse, w.sketch)
    in_bytes = 2 * B * H * T * d * esize
    packed_bytes = 2 * B * H * T * rec
    footprint = in_bytes + 2 * H * cap * rec
    R = args.copies or max(3, math.ceil((1 << 30) / footprint))

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    Kn, Vn, Qn = W.kv_batch(w, 0), W.kv_batch(w, 1), W.queries(w)
    K0, V0 = dev(Kn), dev(Vn)
    Ks, Vs = [K0] + [K0.clone() for _ in range(R - 1)], [V0] + [V0.clone() for _ in range(R - 1)]
    caches = [s.new_caches(cap) for _ in range(R)]
    Q = dev(Qn)
    dst = torch.from_numpy(starts).cuda()
    st_d = torch.from_numpy(starts).cuda()
    ln_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    max_len = int(lens.max())
    ws = s.workspace(B, max_len)
    out = torch.empty(B, w.n_q_heads, d, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def step(i, evs=None):
        r = i % R
        kc, vc = caches[r]
        if evs is not None:
            evs[0].record(stream)
        s.quantize(Ks[r], Vs[r], dst, kc, vc, stream=stream)   # one launch: K and V tiles
        if evs is not None:
            evs[1].record(stream)
        kd, vd = caches[(r + R // 2) % R]
        s.decode(Q, st_d, ln_d, max_len, kd, vd, out=out, workspace=ws, stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(R):          # populate every cache copy
        step(i)
    qt, dt_, wall = timed_steps(args, step)
    assert torch.isfinite(out).all(), "decode produced non-finite output"

    q_avg, d_avg = float(qt.mean()), float(dt_.mean())
    # one launch of the quantize kernel: at d = 128 K and V share one launch (the
    # same spec); at d = 256 the call makes one launch per tensor
    nql = 1 if d == 128 else 2
    ql_avg = q_avg / nql
    q_bytes = in_bytes + packed_bytes
    q_flops = 2 * B * H * T * 4 * d * d           # two d x d contractions per vector
    roof_dec = roofline_decode(w, packed_bytes, d_avg)
    # quantize: the bound at algorithmic cost is the larger of the bytes at HBM peak
    # and the two contractions at bf16 matrix peak (HBM at d = 128, MFMA at d = 256)
    pieces = 6 if d == 128 or w.bits_mse == 3 else 5
    note = (f"algorithmic 4 d^2 flops per vector; executed as {pieces} bf16 piece products per vector "
            f"({pieces - 3} for Pi x, 3 for the sketch)")
    qkern = "quantize_mfma" if d == 128 else "quantize_wide"
    ql_bytes, ql_flops = q_bytes / nql, q_flops // nql
    ql_gbs, ql_tf = ql_bytes / ql_avg / 1e9, ql_flops / ql_avg / 1e12
    q_traffic = traffic_for([("quantize", 1)], w.name)
    hbm_view = {"achieved": ql_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ql_gbs / HBM_PEAK_GBS}
    mfma_view = {"achieved": ql_tf, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": ql_tf / BF16_MFMA_PEAK_TFLOPS, "flops_per_launch": ql_flops, "note": note}
    kdesc = (f"{qkern}: one launch for K and V, {2 * B * H * T} vectors" if nql == 1 else
             f"{qkern}: one launch per tensor (two per call), {B * H * T} vectors")
    if ql_flops / (BF16_MFMA_PEAK_TFLOPS * 1e12) > ql_bytes / (HBM_PEAK_GBS * 1e9):
        roof_q = {"bound": "mfma", **{k: v for k, v in mfma_view.items() if k != "note"}, "traffic": q_traffic,
                  "kernel": kdesc, "bytes_per_launch": ql_bytes, "avg_launch_s": ql_avg, "note": note,
                  "hbm": hbm_view}
    else:
        roof_q = {"bound": "hbm", **hbm_view, "traffic": q_traffic, "kernel": kdesc,
                  "bytes_per_launch": ql_bytes, "avg_launch_s": ql_avg, "mfma": mfma_view}
    res = {
        "ms_per_step": wall * 1e3, "value": packed_bytes / d_avg / 1e9,
        "config": {"workload": w.name, "batch": B, "kv_heads": H, "q_heads": w.n_q_heads, "seq_len": T,
                   "head_dim": d, "bits": w.bits, "input_dtype": w.dtype, "rotation_copies": R,
                   "step": "quantize the whole context (K and V), then one decode step"},
        "quantize_tokens_per_s": B * T / q_avg, "quantize_GBps": q_bytes / q_avg / 1e9,
        "decode_call_s": d_avg, "quantize_call_s": q_avg,
        "roofline": roof_q if ql_avg >= d_avg else roof_dec, "roofline_decode": roof_dec,
        "roofline_quantize": roof_q,
    }

    def ctx(b, h):
        return Kn[b, h], Vn[b, h]

    def mse_only(s2):
        kc, vc = s2.new_caches(cap)
        s2.quantize(K0, V0, dst, kc, vc)
        return s2.decode(Q, st_d, ln_d, max_len, kc, vc).cpu().numpy(), kc

    if not args.no_quality:
        res["quality"] = quality_report(w, rot, proj, ctx, Qn, out.cpu().numpy(), mse_only,
                                        sess=s, kc=caches[0][0], starts=starts)
    return res


def bench_decode_step(args, w, s, rot, proj):
    """Workloads 3 and 4: the earlier context of every sequence is quantized as
    untimed setup; a step quantizes each sequence's newest token (K and V of every
    kv head, one tq_quantize_kv call) into its slot and then decodes over the whole
    context, that token included (one tq_decode_attention call)."""
    import torch
    import workloads as W
    B, H, d = w.batch, w.n_kv_heads, w.d
    if w.ragged:
        # the context is len_s prefill tokens; the step appends one new token
        ctx_len = W.seq_lengths(w)
        chunk = lambda t, b, h: W.kv_chunk(w, t, b, h, n_tokens=int(ctx_len[b]))
        new = lambda t, b, h: W.new_tokens(w, t, b, h)[:1]
    else:
        # a sequence's newest token is the last of its seq_len tokens
        ctx_len = np.full(B, w.seq_len - 1, np.int64)
        full = {t: W.kv_batch(w, t) for t in (0, 1)}
        chunk = lambda t, b, h: full[t][b, h, :int(ctx_len[b])]
        new = lambda t, b, h: full[t][b, h, int(ctx_len[b]):int(ctx_len[b]) + 1]
    lens = ctx_len + 1
    starts = W.seq_starts(ctx_len)       # each region padded to 64 slots with room for the new token
    cap = W.capacity(ctx_len)
    rec = packed_record_bytes(d, w.m, w.bits_mse, w.sketch)
    packed_bytes = int(2 * H * lens.sum() * rec)
    R = args.copies or max(3, math.ceil((1 << 30) / packed_bytes))
    Qn = W.queries(w)
    newk = np.stack([np.stack([new(0, b, h) for h in range(H)]) for b in range(B)])   # [B][H][1][d]
    newv = np.stack([np.stack([new(1, b, h) for h in range(H)]) for b in range(B)])

    def dev(a):
        t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
        return t.view(torch.bfloat16) if a.dtype == np.uint16 else t

    Kd_new, Vd_new, Q = dev(newk), dev(newv), dev(Qn)
    dst_new = torch.from_numpy(starts + ctx_len).cuda()
    st_d = torch.from_numpy(starts).cuda()
    ln_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    max_len = int(lens.max())
    stream = torch.cuda.current_stream()

    # every sequence's earlier context in device memory, [1][H][len_s][d] per tensor
    ctx_dev = [(dev(np.stack([chunk(0, b, h) for h in range(H)])[None]),
                dev(np.stack([chunk(1, b, h) for h in range(H)])[None])) for b in range(B)]

    def prefill(sess):
        """Quantize every sequence's earlier context into a fresh pair of caches."""
        kc, vc = sess.new_caches(cap)
        for b in range(B):
            sess.quantize(ctx_dev[b][0], ctx_dev[b][1], st_d[b:b + 1], kc, vc)
        return kc, vc

    caches = [prefill(s) for _ in range(R)]
    torch.cuda.synchronize()
    ws = s.workspace(B, max_len)
    out = torch.empty(B, w.n_q_heads, d, dtype=torch.float32, device="cuda")

    def step(i, evs=None):
        kc, vc = caches[i % R]
        if evs is not None:
            evs[0].record(stream)
        s.quantize(Kd_new, Vd_new, dst_new, kc, vc, stream=stream)   # K and V of the newest token
        if evs is not None:
            evs[1].record(stream)
        s.decode(Q, st_d, ln_d, max_len, kc, vc, out=out, workspace=ws, stream=stream)
        if evs is not None:
            evs[2].record(stream)

    qt, dt_, wall = timed_steps(args, step)
    assert torch.isfinite(out).all(), "decode produced non-finite output"
    q_avg, d_avg = float(qt.mean()), float(dt_.mean())
    roof_dec = roofline_decode(w, packed_bytes, d_avg)
    q_bytes = 2 * B * H * (d * 2 + rec)
    out_sparse = None
    if args.sparse_v > 0:
        out_sparse = torch.empty_like(out)

        def step_sparse(i, evs=None):
            kc, vc = caches[i % R]
            if evs is not None:
                evs[0].record(stream)
                evs[1].record(stream)
            s.decode(Q, st_d, ln_d, max_len, kc, vc, out=out_sparse, workspace=ws, stream=stream,
                     sparse_v=args.sparse_v)
            if evs is not None:
                evs[2].record(stream)

        _, st_, _ = timed_steps(args, step_sparse)
    res = {
        "ms_per_step": wall * 1e3, "value": packed_bytes / d_avg / 1e9,
        "config": {"workload": w.name, "batch": B, "kv_heads": H, "q_heads": w.n_q_heads,
                   "seq_len": int(lens.max()), "total_tokens": int(lens.sum()), "head_dim": d, "bits": w.bits,
                   "input_dtype": w.dtype, "rotation_copies": R,
                   "step": "quantize one new token per sequence (K and V), then one decode step over len + 1"},
        "quantize_tokens_per_s": B / q_avg, "quantize_GBps": q_bytes / q_avg / 1e9,
        "decode_call_s": d_avg, "quantize_call_s": q_avg,
        "roofline": roof_dec, "roofline_decode": roof_dec,
        "roofline_quantize": {"bound": "launch", "kernel": "quantize_mfma: one launch for K and V, "
                              f"{2 * B * H} vectors", "bytes_per_call": q_bytes, "avg_call_s": q_avg,
                              "note": "a few dozen vectors per call: bound by launch latency, not by a roofline"},
    }

    def ctx(b, h):
        return (np.concatenate([chunk(0, b, h), new(0, b, h)]), np.concatenate([chunk(1, b, h), new(1, b, h)]))

    def mse_only(s2):
        kc, vc = prefill(s2)
        s2.quantize(Kd_new, Vd_new, dst_new, kc, vc)
        return s2.decode(Q, st_d, ln_d, max_len, kc, vc).cpu().numpy(), kc

    if not args.no_quality:
        # the key cache of the last timed step
        res["quality"] = quality_report(w, rot, proj, ctx, Qn, out.cpu().numpy(), mse_only, sess=s,
                                        kc=caches[(args.steps - 1) % R][0], starts=starts)
    if out_sparse is not None:
        sp = float(st_.mean())
        res["sparse_v"] = {"tau": args.sparse_v, "decode_call_s": sp, "GBps_of_dense_bytes": packed_bytes / sp / 1e9,
                           "speedup_vs_dense": d_avg / sp,
                           "note": "Sparse V decode: a first pass over the keys finds each head's largest score, "
                                   "then the split pass leaves out the values of positions with weight below tau "
                                   "times the largest (the bytes read are the dense decode's plus the keys again)"}
        if not args.no_quality:
            res["sparse_v"]["quality"] = quality_vs_unquantized(w, ctx, Qn, out_sparse.cpu().numpy())
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--copies", type=int, default=0, help="rotation copies (0: enough for 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true", help="skip the host-side quality report")
    ap.add_argument("--sparse-v", type=float, default=0.0, metavar="TAU",
                    help="also time Sparse V decode (values of positions with weight below TAU times the "
                         "largest left out) on workloads 3 and 4")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only plain 1 GiB device copies (HBM counter calibration)")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/traffic.json from rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--search", action="store_true",
                    help="measure inner-product search over a packed key index instead")
    ap.add_argument("--search-nq", type=lambda v: [int(x) for x in v.split(",")], default=[8, 32],
                    help="query counts of the search measurement (multiples of 8; the last one is the headline)")
    args = ap.parse_args()
    if args.traffic:
        import workloads as W
        write_traffic(*args.traffic, copy_bytes=1 << 30,
                      workload=SEARCH_WORKLOAD if args.search else W.WORKLOADS[args.workload].name)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this hot path runs on one GPU; multi-GPU runs are not part of this build "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from kv_cache_online_amd.session import TQSession

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        copy_calibration()
        return
    if args.search:
        bench_search(args)
        return
    w = W.WORKLOADS[args.workload]
    rot, proj = W.rotation(w.d, w.wid), W.sketch(w.m, w.d, w.wid)
    s = TQSession(w.d, w.n_kv_heads, w.n_q_heads, rot, proj, k_bits=w.bits_mse, v_bits=w.bits_mse,
                  k_sketch=w.sketch, v_sketch=w.sketch)
    run = bench_decode_step if args.workload in (3, 4) else bench_context
    r = run(args, w, s, rot, proj)
    status = int(s.status.item()) & 0xFFFFFFFF
    assert status == 0, f"device status flags {status:#x}"
    copy_gbs = copy_peak_gbs()
    dec_gbs = r.pop("value")
    res = {
        "metric": METRIC, "value": dec_gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r.pop("ms_per_step"), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16+i8",
        "data": "synthetic (seeded Gaussian K/V/Q with per-channel scales and outlier channels)",
        "config": r.pop("config"),
        "decode_pct_hbm_peak": 100 * dec_gbs / HBM_PEAK_GBS,
        "hbm_copy_GBps": copy_gbs, "decode_frac_of_copy": dec_gbs / copy_gbs,
        "compute": "quantize: bf16-piece MFMA, fp32 accumulate; decode: scores on fp6 (query digits) x fp4 "
                   "(key bits) scaled MFMA, fp32 accumulate; values on exact int8 MFMA, int32 accumulate; "
                   "fp32/fp64 softmax and merge",
        **r, "source_hash": source_hash(),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, rot, proj, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
